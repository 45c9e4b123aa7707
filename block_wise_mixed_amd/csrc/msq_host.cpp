// C ABI of the msq library (declared in include/msq.h): argument checks,
// buffer sizing, and dispatch to the gfx950 kernels on the caller's stream.
// Every check runs before the first launch, so a call that returns an error
// leaves its outputs untouched.
#include "msq.h"

#include <hip/hip_runtime.h>

#include <cstring>
#include <vector>

#include "msq_internal.h"

namespace {

using msq::kBlockCols;
using msq::kBlockRows;

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool bits_ok(uint8_t b) {
  return b == 0 || b == 1 || b == 2 || b == 3 || b == 4 || b == 8 || b == 16;
}

msq_status check_shape(int64_t N, int64_t K) {
  if (N <= 0 || K <= 0 || N % kBlockRows != 0 || K % kBlockCols != 0) return MSQ_ERR_SHAPE;
  // block rows, block columns and per-row indices are handled as 32-bit ints
  if (N > (int64_t)0x7FFFFFFF || K > (int64_t)0x7FFFFFFF) return MSQ_ERR_SHAPE;
  if ((N / kBlockRows) * (K / kBlockCols) > (int64_t)0x7FFFFFFF) return MSQ_ERR_SHAPE;
  return MSQ_OK;
}

bool is_permutation(const int32_t* p, int64_t n) {
  std::vector<uint8_t> seen((size_t)n, 0);
  for (int64_t i = 0; i < n; ++i) {
    const int32_t v = p[i];
    if (v < 0 || v >= n || seen[(size_t)v]) return false;
    seen[(size_t)v] = 1;
  }
  return true;
}

msq_status plan_impl(int64_t N, int64_t K, const uint8_t* bits, const int32_t* prow,
                     const int32_t* pcol, msq_sizes* out) {
  msq_status st = check_shape(N, K);
  if (st != MSQ_OK) return st;
  const int64_t nblk = (N / kBlockRows) * (K / kBlockCols);
  msq_sizes s;
  std::memset(&s, 0, sizeof(s));
  int64_t total_bits = 0;
  for (int64_t i = 0; i < nblk; ++i) {
    if (!bits_ok(bits[i])) return MSQ_ERR_BITS;
    s.blocks_per_bits[bits[i]]++;
    total_bits += bits[i];
  }
  if (!is_permutation(prow, N) || !is_permutation(pcol, K)) return MSQ_ERR_PERM;
  if (total_bits > (int64_t)0xFFFFFFFE) return MSQ_ERR_SHAPE;  // offsets are 32-bit KiB counts
  s.code_bytes = 1024 * total_bits;
  s.scale_bytes = 4 * N * (K / kBlockCols);
  s.zero_bytes = N * (K / kBlockCols);
  s.offset_bytes = 4 * nblk;
  s.mean_bits = (double)total_bits / (double)nblk;
  *out = s;
  return MSQ_OK;
}

msq_status weight_ptrs_ok(const msq_weight* w) {
  if (!w) return MSQ_ERR_INVALID_ARG;
  if (!w->bits || !w->perm_row || !w->perm_col || !w->block_offset || !w->scale || !w->zero)
    return MSQ_ERR_INVALID_ARG;
  if (!w->codes && w->code_bytes > 0) return MSQ_ERR_INVALID_ARG;
  if (w->tile16_blocks < 0) return MSQ_ERR_INVALID_ARG;
  if (w->codes && !aligned(w->codes, 256)) return MSQ_ERR_INVALID_ARG;
  if (!aligned(w->perm_row, 4) || !aligned(w->perm_col, 16) || !aligned(w->block_offset, 4) ||
      !aligned(w->scale, 16) || !aligned(w->zero, 16))
    return MSQ_ERR_INVALID_ARG;
  return check_shape(w->N, w->K);
}

msq::WeightView view_of(const msq_weight* w) {
  msq::WeightView v;
  v.N = w->N;
  v.K = w->K;
  v.NBr = (int)(w->N / kBlockRows);
  v.NBc = (int)(w->K / kBlockCols);
  v.bits = w->bits;
  v.perm_row = w->perm_row;
  v.perm_col = w->perm_col;
  v.block_offset = w->block_offset;
  v.codes = w->codes;
  v.scale = w->scale;
  v.zero = w->zero;
  v.has16 = w->tile16_blocks > 0 ? 1 : 0;
  return v;
}

size_t workspace_for(int64_t M, int64_t N, int64_t K, msq_kernel kernel) {
  if (M <= 0) return 0;
  const size_t gemv = M <= MSQ_GEMV_MAX_M ? msq::plan_gemv(M, N, K).workspace : 0;
  const size_t gemm = msq::gemm_workspace_bytes(M, N, K);
  switch (kernel) {
    case MSQ_KERNEL_GEMV: return gemv;
    case MSQ_KERNEL_GEMM: return gemm;
    default: return M <= MSQ_AUTO_GEMV_MAX_M ? gemv : gemm;
  }
}

}  // namespace

extern "C" {

msq_status msq_plan(int64_t N, int64_t K, const uint8_t* bits_host, const int32_t* perm_row_host,
                    const int32_t* perm_col_host, msq_sizes* out) {
  if (!bits_host || !perm_row_host || !perm_col_host || !out) return MSQ_ERR_INVALID_ARG;
  return plan_impl(N, K, bits_host, perm_row_host, perm_col_host, out);
}

msq_status msq_quantize_pack(const uint16_t* W_bf16, const msq_weight* w, hipStream_t stream) {
  if (!W_bf16 || !aligned(W_bf16, 16)) return MSQ_ERR_INVALID_ARG;
  msq_status st = weight_ptrs_ok(w);
  if (st != MSQ_OK) return st;
  const int64_t N = w->N, K = w->K;
  const int64_t nblk = (N / kBlockRows) * (K / kBlockCols);
  // Read the descriptor's bit map and permutations back and validate them as
  // msq_plan does, so the kernels below can never index out of bounds.
  std::vector<uint8_t> bits((size_t)nblk);
  std::vector<int32_t> prow((size_t)N), pcol((size_t)K);
  if (hipMemcpyAsync(bits.data(), w->bits, (size_t)nblk, hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipMemcpyAsync(prow.data(), w->perm_row, (size_t)N * 4, hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipMemcpyAsync(pcol.data(), w->perm_col, (size_t)K * 4, hipMemcpyDeviceToHost, stream) != hipSuccess ||
      hipStreamSynchronize(stream) != hipSuccess)
    return MSQ_ERR_HIP;
  msq_sizes sz;
  st = plan_impl(N, K, bits.data(), prow.data(), pcol.data(), &sz);
  if (st != MSQ_OK) return st;
  if (w->code_bytes < sz.code_bytes) return MSQ_ERR_BUFFER_TOO_SMALL;
  if (w->tile16_blocks != sz.blocks_per_bits[16]) return MSQ_ERR_INVALID_ARG;
  if (hipError_t e = msq::launch_block_offsets(w->bits, nblk, w->block_offset, stream); e != hipSuccess)
    return MSQ_ERR_HIP;
  if (hipError_t e = msq::launch_pack(W_bf16, N, K, w->bits, w->perm_row, w->perm_col,
                                      w->block_offset, w->codes, w->scale, w->zero, stream);
      e != hipSuccess)
    return MSQ_ERR_HIP;
  return MSQ_OK;
}

size_t msq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (check_shape(N, K) != MSQ_OK || M <= 0) return 0;
  // enough for either kernel, so msq_gemm_ex may pick any of them
  const size_t a = workspace_for(M, N, K, MSQ_KERNEL_GEMV);
  const size_t b = workspace_for(M, N, K, MSQ_KERNEL_GEMM);
  return a > b ? a : b;
}

msq_status msq_gemm_ex(const uint16_t* x_bf16, int64_t M, const msq_weight* w, float* y,
                       void* workspace, size_t workspace_bytes, msq_kernel kernel,
                       hipStream_t stream) {
  if (kernel != MSQ_KERNEL_AUTO && kernel != MSQ_KERNEL_GEMV && kernel != MSQ_KERNEL_GEMM)
    return MSQ_ERR_INVALID_ARG;
  msq_status st = weight_ptrs_ok(w);
  if (st != MSQ_OK) return st;
  if (M < 0) return MSQ_ERR_SHAPE;
  if (M == 0) return MSQ_OK;
  if (M > (int64_t)0x7FFFFFFF / 2) return MSQ_ERR_SHAPE;
  if (!x_bf16 || !y || !aligned(x_bf16, 16) || !aligned(y, 4)) return MSQ_ERR_INVALID_ARG;
  if (kernel == MSQ_KERNEL_AUTO) kernel = M <= MSQ_AUTO_GEMV_MAX_M ? MSQ_KERNEL_GEMV : MSQ_KERNEL_GEMM;
  if (kernel == MSQ_KERNEL_GEMV && M > MSQ_GEMV_MAX_M) return MSQ_ERR_UNSUPPORTED;
  const size_t need = workspace_for(M, w->N, w->K, kernel);
  if (need > 0 && (!workspace || !aligned(workspace, 256))) return MSQ_ERR_INVALID_ARG;
  if (workspace_bytes < need) return MSQ_ERR_BUFFER_TOO_SMALL;
  const msq::WeightView v = view_of(w);
  hipError_t e;
  const uint16_t* xr = nullptr;  // reordered x left in the workspace (M > 1)
  bool pass16 = w->tile16_blocks > 0;  // 16-bit blocks left to k_tile16
  if (kernel == MSQ_KERNEL_GEMV) {
    const msq::GemvPlan p = msq::plan_gemv(M, w->N, w->K);
    e = msq::launch_gemv(x_bf16, M, v, y, workspace, p, stream);
    xr = msq::gemv_reordered_x(workspace, p, M, w->N);
  } else {
    e = msq::launch_gemm(x_bf16, M, v, y, workspace, stream);
    xr = reinterpret_cast<const uint16_t*>(workspace);
    pass16 = pass16 && !msq::gemm_handles_tile16();
  }
  if (e == hipSuccess && pass16) e = msq::launch_tile16(x_bf16, xr, M, v, y, stream);
  return e == hipSuccess ? MSQ_OK : MSQ_ERR_HIP;
}

msq_status msq_gemm(const uint16_t* x_bf16, int64_t M, const msq_weight* w, float* y,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return msq_gemm_ex(x_bf16, M, w, y, workspace, workspace_bytes, MSQ_KERNEL_AUTO, stream);
}

size_t msq_gemm_group_workspace_bytes(int64_t M, const msq_weight* const* w, int count) {
  if (!w || count < 1 || count > MSQ_GROUP_MAX || M <= 0) return 0;
  msq::WeightView v[MSQ_GROUP_MAX];
  size_t most = 0;
  for (int i = 0; i < count; ++i) {
    if (!w[i] || check_shape(w[i]->N, w[i]->K) != MSQ_OK) return 0;
    v[i] = view_of(w[i]);
    const size_t one = msq_gemm_workspace_bytes(M, w[i]->N, w[i]->K);
    most = one > most ? one : most;
  }
  // M == 1 and M > 16: every matrix keeps its own workspace (one launch for
  // all, or split-K single calls); 2 .. 16: the matrices run one after the
  // other
  if (M == 1) return msq::gemv_group_workspace_m1(v, count);
  if (M > MSQ_AUTO_GEMV_MAX_M) return msq::gemm_group_workspace_bytes(M, v, count);
  return most;
}

msq_status msq_gemm_group(const uint16_t* const* x_bf16, int64_t M, const msq_weight* const* w,
                          float* const* y, int count, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  static_assert(MSQ_GROUP_MAX == msq::kGemvGroupMax, "group size of the header and the kernels");
  if (!x_bf16 || !w || !y || count < 1 || count > MSQ_GROUP_MAX) return MSQ_ERR_INVALID_ARG;
  for (int i = 0; i < count; ++i) {
    const msq_status st = weight_ptrs_ok(w[i]);
    if (st != MSQ_OK) return st;
    if (!x_bf16[i] || !y[i] || !aligned(x_bf16[i], 16) || !aligned(y[i], 4))
      return MSQ_ERR_INVALID_ARG;
  }
  if (M < 0) return MSQ_ERR_SHAPE;
  if (M == 0) return MSQ_OK;
  if (M > (int64_t)0x7FFFFFFF / 2) return MSQ_ERR_SHAPE;
  if (M != 1 && M <= MSQ_AUTO_GEMV_MAX_M) {
    // one matrix after the other, sharing the workspace (ordered on stream)
    for (int i = 0; i < count; ++i) {
      const msq_status st = msq_gemm(x_bf16[i], M, w[i], y[i], workspace, workspace_bytes, stream);
      if (st != MSQ_OK) return st;
    }
    return MSQ_OK;
  }
  const size_t need = msq_gemm_group_workspace_bytes(M, w, count);
  if (need > 0 && (!workspace || !aligned(workspace, 256))) return MSQ_ERR_INVALID_ARG;
  if (workspace_bytes < need) return MSQ_ERR_BUFFER_TOO_SMALL;
  msq::WeightView v[MSQ_GROUP_MAX];
  for (int i = 0; i < count; ++i) v[i] = view_of(w[i]);
  hipError_t e = M == 1 ? msq::launch_gemv_group_m1(x_bf16, v, y, count, workspace, stream)
                        : msq::launch_gemm_group(x_bf16, M, v, y, count, workspace, stream);
  // M > 16: job i's reordered x starts its workspace share
  const uint8_t* share = reinterpret_cast<const uint8_t*>(workspace);
  const bool gemm16 = M > 1 && msq::gemm_handles_tile16();
  for (int i = 0; i < count && e == hipSuccess; ++i) {
    const uint16_t* xr = M == 1 ? nullptr : reinterpret_cast<const uint16_t*>(share);
    if (w[i]->tile16_blocks > 0 && !gemm16)
      e = msq::launch_tile16(x_bf16[i], xr, M, v[i], y[i], stream);
    share += (msq::gemm_workspace_bytes(M, w[i]->N, w[i]->K) + 255) & ~(size_t)255;
  }
  return e == hipSuccess ? MSQ_OK : MSQ_ERR_HIP;
}

const char* msq_status_string(msq_status s) {
  switch (s) {
    case MSQ_OK: return "success";
    case MSQ_ERR_INVALID_ARG: return "invalid argument (null, misaligned pointer or bad enum)";
    case MSQ_ERR_SHAPE: return "bad shape (N % 64, K % 128, sizes out of range or M < 0)";
    case MSQ_ERR_BITS: return "bit map entry outside {0,1,2,3,4,8,16}";
    case MSQ_ERR_PERM: return "perm_row or perm_col is not a permutation";
    case MSQ_ERR_BUFFER_TOO_SMALL: return "buffer too small";
    case MSQ_ERR_HIP: return "HIP runtime or launch error";
    case MSQ_ERR_UNSUPPORTED: return "unsupported configuration";
  }
  return "unknown status";
}

int msq_format_version(void) { return MSQ_FORMAT_VERSION; }

}  // extern "C"
