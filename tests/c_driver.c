/* One drop layer driven from plain C through include/uniprefill.h, with device
 * buffers from the HIP runtime and nothing else in the process (no Python, no
 * torch): up_select_blocks -> up_compact (one row buffer) -> up_update_metadata
 * -> up_scatter_back.  tests/test_gpu_c_driver.py writes the inputs (seeded
 * synthetic workload), runs this program as a child process and checks what it
 * writes against the CPU oracle.
 *
 *   c_driver IN OUT
 *
 * IN (little-endian): int32 magic 0x31435055, R, T, Hq, Hkv, d, G, A, n,
 * row_bytes, layer, num_layers; float64 p; int32 cu_seqlens[R+1];
 * int32 seq_lens[R]; uint16 q[T*Hq*d]; uint16 k[T*Hkv*d]; uint8 hidden[T*row_bytes].
 *
 * OUT: int32 status[4] (select, compact, metadata, scatter); int64 max_blocks;
 * float32 block_scores[max_blocks]; int32 block_offsets[R+1];
 * uint8 keep_block[max_blocks]; uint8 keep_mask[T]; int32 kept[R];
 * int32 cu_out[R+1]; int32 index_out[T]; uint8 hidden_out[T*row_bytes];
 * int32 seq_lens[R]; int32 num_actual_tokens; int32 drop_count[R];
 * int32 drop_layer[R*2]; int32 drop_len[R*2]; int32 seqused_base[num_layers*R];
 * uint8 full[T*row_bytes] (0xEE everywhere, then the scatter-back of hidden_out).
 * Exit status 0 when every call returned UP_OK and no HIP call failed.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <hip/hip_runtime_api.h>

#include "uniprefill.h"

#define MAX_DROPS 2

#define HIP_CHECK(call)                                                          \
  do {                                                                           \
    hipError_t e_ = (call);                                                      \
    if (e_ != hipSuccess) {                                                      \
      fprintf(stderr, "%s:%d %s: %s\n", __FILE__, __LINE__, #call, hipGetErrorString(e_)); \
      exit(2);                                                                   \
    }                                                                            \
  } while (0)

static void read_exact(FILE* f, void* dst, size_t bytes) {
  if (bytes && fread(dst, 1, bytes, f) != bytes) {
    fprintf(stderr, "short input\n");
    exit(2);
  }
}

static void write_exact(FILE* f, const void* src, size_t bytes) {
  if (bytes && fwrite(src, 1, bytes, f) != bytes) {
    fprintf(stderr, "short write\n");
    exit(2);
  }
}

static void* dev_alloc(size_t bytes) {
  void* p = NULL;
  HIP_CHECK(hipMalloc(&p, bytes ? bytes : 256));
  return p;
}

static void* host_alloc(size_t bytes) {
  void* p = malloc(bytes ? bytes : 1);
  if (p == NULL) {
    fprintf(stderr, "out of host memory\n");
    exit(2);
  }
  return p;
}

/* copy `bytes` from device to host and append them to the output */
static void dump(FILE* f, const void* dev, size_t bytes) {
  void* h = host_alloc(bytes);
  HIP_CHECK(hipMemcpy(h, dev, bytes, hipMemcpyDeviceToHost));
  write_exact(f, h, bytes);
  free(h);
}

int main(int argc, char** argv) {
  if (argc != 3) {
    fprintf(stderr, "usage: %s IN OUT\n", argv[0]);
    return 2;
  }
  FILE* in = fopen(argv[1], "rb");
  if (in == NULL) {
    perror(argv[1]);
    return 2;
  }
  int32_t hdr[12];
  double p;
  read_exact(in, hdr, sizeof(hdr));
  read_exact(in, &p, sizeof(p));
  if (hdr[0] != 0x31435055) {
    fprintf(stderr, "bad magic\n");
    return 2;
  }
  const int32_t R = hdr[1], T = hdr[2], hq = hdr[3], hkv = hdr[4], d = hdr[5], G = hdr[6], A = hdr[7],
                n = hdr[8], rb = hdr[9], layer = hdr[10], num_layers = hdr[11];
  if (R < 1 || T < 1 || hq < 1 || hkv < 1 || d < 1 || rb < 16 || num_layers < 1) {
    fprintf(stderr, "bad header\n");
    return 2;
  }
  const size_t q_bytes = (size_t)T * hq * d * 2, k_bytes = (size_t)T * hkv * d * 2;
  const size_t h_bytes = (size_t)T * rb;
  int32_t* cu_h = host_alloc(sizeof(int32_t) * (R + 1));
  int32_t* seq_h = host_alloc(sizeof(int32_t) * R);
  void* q_h = host_alloc(q_bytes);
  void* k_h = host_alloc(k_bytes);
  void* hid_h = host_alloc(h_bytes);
  read_exact(in, cu_h, sizeof(int32_t) * (R + 1));
  read_exact(in, seq_h, sizeof(int32_t) * R);
  read_exact(in, q_h, q_bytes);
  read_exact(in, k_h, k_bytes);
  read_exact(in, hid_h, h_bytes);
  fclose(in);

  hipStream_t stream;
  HIP_CHECK(hipStreamCreate(&stream));

  up_select_params prm;
  memset(&prm, 0, sizeof(prm));
  prm.num_heads_q = hq;
  prm.num_heads_kv = hkv;
  prm.head_dim = d;
  prm.block_size = G;
  prm.num_sink = A;
  prm.window = n;
  prm.top_p = p;
  prm.softmax_scale = 0.0f;
  prm.flags = 0u;

  const int64_t max_blocks = up_max_blocks(G, R, T);
  const size_t sel_ws = up_select_workspace_bytes(&prm, R, T);
  const size_t cmp_ws = up_compact_workspace_bytes(R, T);
  if (max_blocks < 1 || sel_ws == 0 || cmp_ws == 0) {
    fprintf(stderr, "sizing failed\n");
    return 2;
  }

  void* q = dev_alloc(q_bytes);
  void* k = dev_alloc(k_bytes);
  int32_t* cu = dev_alloc(sizeof(int32_t) * (R + 1));
  void* hidden = dev_alloc(h_bytes);
  float* scores = dev_alloc(sizeof(float) * max_blocks);
  int32_t* boff = dev_alloc(sizeof(int32_t) * (R + 1));
  uint8_t* keep_block = dev_alloc((size_t)max_blocks);
  uint8_t* mask = dev_alloc((size_t)T);
  int32_t* kept = dev_alloc(sizeof(int32_t) * R);
  void* sel_w = dev_alloc(sel_ws);
  void* hidden_c = dev_alloc(h_bytes);
  int32_t* index_out = dev_alloc(sizeof(int32_t) * T);
  int32_t* cu_out = dev_alloc(sizeof(int32_t) * (R + 1));
  void* cmp_w = dev_alloc(cmp_ws);
  int32_t* seq = dev_alloc(sizeof(int32_t) * R);
  int32_t* nat = dev_alloc(sizeof(int32_t));
  int32_t* dcount = dev_alloc(sizeof(int32_t) * R);
  int32_t* dlayer = dev_alloc(sizeof(int32_t) * R * MAX_DROPS);
  int32_t* dlen = dev_alloc(sizeof(int32_t) * R * MAX_DROPS);
  int32_t* sbase = dev_alloc(sizeof(int32_t) * R * num_layers);
  void* full = dev_alloc(h_bytes);

  HIP_CHECK(hipMemcpy(q, q_h, q_bytes, hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(k, k_h, k_bytes, hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(cu, cu_h, sizeof(int32_t) * (R + 1), hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(hidden, hid_h, h_bytes, hipMemcpyHostToDevice));
  HIP_CHECK(hipMemcpy(seq, seq_h, sizeof(int32_t) * R, hipMemcpyHostToDevice));
  for (int32_t l = 0; l < num_layers; ++l)
    HIP_CHECK(hipMemcpy(sbase + (size_t)l * R, seq_h, sizeof(int32_t) * R, hipMemcpyHostToDevice));
  HIP_CHECK(hipMemset(dcount, 0, sizeof(int32_t) * R));
  HIP_CHECK(hipMemset(dlayer, 0xFF, sizeof(int32_t) * R * MAX_DROPS));
  HIP_CHECK(hipMemset(dlen, 0xFF, sizeof(int32_t) * R * MAX_DROPS));
  HIP_CHECK(hipMemset(nat, 0, sizeof(int32_t)));
  HIP_CHECK(hipMemset(full, 0xEE, h_bytes));
  HIP_CHECK(hipMemset(scores, 0, sizeof(float) * max_blocks));
  HIP_CHECK(hipMemset(keep_block, 0, (size_t)max_blocks));
  HIP_CHECK(hipMemset(hidden_c, 0, h_bytes));
  HIP_CHECK(hipMemset(index_out, 0xFF, sizeof(int32_t) * T));
  HIP_CHECK(hipDeviceSynchronize());

  int32_t status[4];
  status[0] = up_select_blocks(&prm, q, (int64_t)hq * d, k, (int64_t)hkv * d, cu, R, T, NULL, scores, boff,
                               keep_block, mask, kept, sel_w, sel_ws, stream);
  const void* src[1] = {hidden};
  void* dst[1] = {hidden_c};
  const int64_t row_bytes[1] = {rb};
  status[1] = up_compact(mask, cu, R, T, 1, src, dst, row_bytes, NULL, index_out, cu_out, cmp_w, cmp_ws,
                         stream);
  status[2] = up_update_metadata(layer, num_layers, R, cu, cu_out, seq, nat, dcount, dlayer, dlen, MAX_DROPS,
                                 sbase, stream);
  status[3] = up_scatter_back(hidden_c, rb, index_out, cu_out, R, T, full, T, stream);
  HIP_CHECK(hipStreamSynchronize(stream));

  FILE* out = fopen(argv[2], "wb");
  if (out == NULL) {
    perror(argv[2]);
    return 2;
  }
  write_exact(out, status, sizeof(status));
  write_exact(out, &max_blocks, sizeof(max_blocks));
  dump(out, scores, sizeof(float) * max_blocks);
  dump(out, boff, sizeof(int32_t) * (R + 1));
  dump(out, keep_block, (size_t)max_blocks);
  dump(out, mask, (size_t)T);
  dump(out, kept, sizeof(int32_t) * R);
  dump(out, cu_out, sizeof(int32_t) * (R + 1));
  dump(out, index_out, sizeof(int32_t) * T);
  dump(out, hidden_c, h_bytes);
  dump(out, seq, sizeof(int32_t) * R);
  dump(out, nat, sizeof(int32_t));
  dump(out, dcount, sizeof(int32_t) * R);
  dump(out, dlayer, sizeof(int32_t) * R * MAX_DROPS);
  dump(out, dlen, sizeof(int32_t) * R * MAX_DROPS);
  dump(out, sbase, sizeof(int32_t) * R * num_layers);
  dump(out, full, h_bytes);
  fclose(out);

  void* bufs[] = {q, k, cu, hidden, scores, boff, keep_block, mask, kept, sel_w, hidden_c, index_out,
                  cu_out, cmp_w, seq, nat, dcount, dlayer, dlen, sbase, full};
  for (size_t i = 0; i < sizeof(bufs) / sizeof(bufs[0]); ++i) HIP_CHECK(hipFree(bufs[i]));
  HIP_CHECK(hipStreamDestroy(stream));
  free(cu_h);
  free(seq_h);
  free(q_h);
  free(k_h);
  free(hid_h);
  for (int i = 0; i < 4; ++i)
    if (status[i] != UP_OK) {
      fprintf(stderr, "call %d returned %d (%s)\n", i, status[i], up_status_string((up_status)status[i]));
      return 1;
    }
  printf("ok\n");
  return 0;
}
