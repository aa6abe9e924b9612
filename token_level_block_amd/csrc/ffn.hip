// A downstream sublayer on the retained rows: the gated FFN of the LLaMA
// family, y = (silu(x Wg^T) * (x Wu^T)) Wd^T, token by token (UniPrefill
// Sec. 3.4 Eq. 7: after a drop every later sublayer maps only the retained
// rows; Eq. 9-10: that is where the saving comes from).
//
// The two projections are plain bf16 GEMMs with fp32 accumulation and run in
// hipBLASLt.  The weights are in the [out_features][in_features] layout of a
// linear layer, so with hipBLASLt's column-major view each product is
//   D (N x rows) = op_T(A = W, K x N) * op_N(B = X^T, K x rows),
// which leaves D as the row-major [rows][N] output.  Between them,
// swiglu_kernel reads the [rows][2F] gate/up product (gate columns first) and
// writes h = silu(gate) * up as bf16 [rows][F], eight channels per thread
// with 16-byte accesses, in fp32 arithmetic.
#include <hipblaslt/hipblaslt.h>

#include "../../include/uniprefill.h"
#include "common.h"

namespace up {

constexpr int kSwigluThreads = 256;
constexpr size_t kLtWorkspace = size_t(64) << 20;   // hipBLASLt scratch inside the caller's workspace

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ float silu_f32(float g) {
  // g * sigmoid(g) = g / (1 + 2^(-g log2 e)); large negative g gives -0
  const float e = __builtin_amdgcn_exp2f(-g * 1.4426950408889634f);
  return g * __builtin_amdgcn_rcpf(1.0f + e);
}

__global__ __launch_bounds__(kSwigluThreads) void swiglu_kernel(const __bf16* __restrict__ gu,
                                                                __bf16* __restrict__ h, int64_t rows,
                                                                int64_t F) {
  const int64_t per_row = F / 8;
  const int64_t t = (int64_t)blockIdx.x * kSwigluThreads + threadIdx.x;
  if (t >= rows * per_row) return;
  const int64_t r = t / per_row, c = (t - r * per_row) * 8;
  const bf16x8 g = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(gu + r * 2 * F + c));
  const bf16x8 u = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(gu + r * 2 * F + F + c));
  bf16x8 o;
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = (__bf16)(silu_f32((float)g[i]) * (float)u[i]);
  *reinterpret_cast<bf16x8*>(h + r * F + c) = o;
}

}  // namespace up

namespace {

size_t align_up256(size_t x) { return (x + 255) / 256 * 256; }

struct GemmCache {
  int64_t rows = -1;
  hipblasLtMatmulAlgo_t algo{};
};

}  // namespace

struct up_ffn {
  int32_t D = 0, F = 0;
  hipblasLtHandle_t lt = nullptr;
  hipblasLtMatmulDesc_t desc = nullptr;
  hipblasLtMatmulPreference_t pref = nullptr;
  GemmCache cache[2];   // the gate/up and the down projection, for the last row count
};

namespace {

// D (n x rows, ld n) = W^T-view product: A = W (k x n column-major, ld k), B = X (k x rows, ld k)
hipblasStatus_t run_gemm(up_ffn* f, int which, const void* W, const void* X, void* Dm, int64_t n, int64_t k,
                         int64_t rows, void* ws, hipStream_t stream) {
  hipblasLtMatrixLayout_t la = nullptr, lb = nullptr, ld = nullptr;
  hipblasStatus_t st = hipblasLtMatrixLayoutCreate(&la, HIP_R_16BF, (uint64_t)k, (uint64_t)n, k);
  if (st == HIPBLAS_STATUS_SUCCESS) st = hipblasLtMatrixLayoutCreate(&lb, HIP_R_16BF, (uint64_t)k, (uint64_t)rows, k);
  if (st == HIPBLAS_STATUS_SUCCESS) st = hipblasLtMatrixLayoutCreate(&ld, HIP_R_16BF, (uint64_t)n, (uint64_t)rows, n);
  GemmCache& c = f->cache[which];
  if (st == HIPBLAS_STATUS_SUCCESS && c.rows != rows) {
    hipblasLtMatmulHeuristicResult_t res[1];
    int found = 0;
    st = hipblasLtMatmulAlgoGetHeuristic(f->lt, f->desc, la, lb, ld, ld, f->pref, 1, res, &found);
    if (st == HIPBLAS_STATUS_SUCCESS && found < 1) st = HIPBLAS_STATUS_NOT_SUPPORTED;
    if (st == HIPBLAS_STATUS_SUCCESS) {
      c.algo = res[0].algo;
      c.rows = rows;
    }
  }
  if (st == HIPBLAS_STATUS_SUCCESS) {
    const float alpha = 1.0f, beta = 0.0f;
    st = hipblasLtMatmul(f->lt, f->desc, &alpha, W, la, X, lb, &beta, Dm, ld, Dm, ld, &c.algo, ws,
                         up::kLtWorkspace, stream);
  }
  if (la) hipblasLtMatrixLayoutDestroy(la);
  if (lb) hipblasLtMatrixLayoutDestroy(lb);
  if (ld) hipblasLtMatrixLayoutDestroy(ld);
  return st;
}

}  // namespace

extern "C" {

up_status up_ffn_create(int32_t hidden, int32_t intermediate, up_ffn** out) {
  if (out == nullptr) return UP_ERR_NULL;
  *out = nullptr;
  if (hidden < 8 || intermediate < 8 || hidden % 8 != 0 || intermediate % 8 != 0) return UP_ERR_PARAM;
  up_ffn* f = new up_ffn;
  f->D = hidden;
  f->F = intermediate;
  const hipblasOperation_t ta = HIPBLAS_OP_T, tb = HIPBLAS_OP_N;
  const uint64_t wsb = up::kLtWorkspace;
  bool ok = hipblasLtCreate(&f->lt) == HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatmulDescCreate(&f->desc, HIPBLAS_COMPUTE_32F, HIP_R_32F) == HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatmulDescSetAttribute(f->desc, HIPBLASLT_MATMUL_DESC_TRANSA, &ta, sizeof(ta)) ==
                HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatmulDescSetAttribute(f->desc, HIPBLASLT_MATMUL_DESC_TRANSB, &tb, sizeof(tb)) ==
                HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatmulPreferenceCreate(&f->pref) == HIPBLAS_STATUS_SUCCESS &&
            hipblasLtMatmulPreferenceSetAttribute(f->pref, HIPBLASLT_MATMUL_PREF_MAX_WORKSPACE_BYTES, &wsb,
                                                  sizeof(wsb)) == HIPBLAS_STATUS_SUCCESS;
  if (!ok) {
    up_ffn_destroy(f);
    return UP_ERR_HIP;
  }
  *out = f;
  return UP_OK;
}

void up_ffn_destroy(up_ffn* f) {
  if (f == nullptr) return;
  if (f->pref) hipblasLtMatmulPreferenceDestroy(f->pref);
  if (f->desc) hipblasLtMatmulDescDestroy(f->desc);
  if (f->lt) hipblasLtDestroy(f->lt);
  delete f;
}

size_t up_ffn_workspace_bytes(const up_ffn* f, int64_t rows) {
  if (f == nullptr || rows < 0) return 0;
  return align_up256((size_t)rows * 2 * f->F * 2) + align_up256((size_t)rows * f->F * 2) + up::kLtWorkspace;
}

up_status up_ffn_forward(up_ffn* f, const void* x, int64_t rows, const void* w_gate_up, const void* w_down,
                         void* y, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (f == nullptr) return UP_ERR_NULL;
  if (rows < 0) return UP_ERR_SHAPE;
  if (rows == 0) return UP_OK;
  if (x == nullptr || w_gate_up == nullptr || w_down == nullptr || y == nullptr || workspace == nullptr)
    return UP_ERR_NULL;
  if (((uintptr_t)x | (uintptr_t)w_gate_up | (uintptr_t)w_down | (uintptr_t)y | (uintptr_t)workspace) % 16 != 0)
    return UP_ERR_ALIGN;
  // the activation kernel's grid (eight channels per thread) must fit 32 bits
  if (rows > (int64_t)UINT32_MAX / (f->F / 8) * up::kSwigluThreads / 2) return UP_ERR_SHAPE;
  if (workspace_bytes < up_ffn_workspace_bytes(f, rows)) return UP_ERR_WORKSPACE;
  const int64_t D = f->D, F = f->F;
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  __bf16* gu = reinterpret_cast<__bf16*>(ws);
  __bf16* h = reinterpret_cast<__bf16*>(ws + align_up256((size_t)rows * 2 * F * 2));
  void* lt_ws = ws + align_up256((size_t)rows * 2 * F * 2) + align_up256((size_t)rows * F * 2);
  if (run_gemm(f, 0, w_gate_up, x, gu, 2 * F, D, rows, lt_ws, stream) != HIPBLAS_STATUS_SUCCESS)
    return UP_ERR_HIP;
  const int64_t threads = rows * (F / 8);
  hipLaunchKernelGGL(up::swiglu_kernel, dim3((unsigned)((threads + up::kSwigluThreads - 1) / up::kSwigluThreads)),
                     dim3(up::kSwigluThreads), 0, stream, gu, h, rows, F);
  if (hipGetLastError() != hipSuccess) return UP_ERR_HIP;
  if (run_gemm(f, 1, w_down, h, y, D, F, rows, lt_ws, stream) != HIPBLAS_STATUS_SUCCESS) return UP_ERR_HIP;
  return UP_OK;
}

}  // extern "C"
