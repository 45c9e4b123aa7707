// C ABI of the msq library (declared in include/msq.h): argument checks,
// buffer sizing, and dispatch to the gfx950 kernels on the caller's stream.
// Every check runs before the first launch, so a call that returns an error
// leaves its outputs untouched.
#include "msq.h"

#include <hip/hip_runtime.h>

#include <cstring>
#include <mutex>
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

// Options of the public struct (NULL = automatic); false for bad values.
bool options_of(const msq_options* o, msq::Options& out) {
  out = msq::Options{};
  if (!o) return true;
  if (o->kernel != MSQ_KERNEL_AUTO && o->kernel != MSQ_KERNEL_GEMV && o->kernel != MSQ_KERNEL_GEMM)
    return false;
  if (o->gemv_split < 0 || o->gemm_split < 0) return false;
  if (o->gemv_waves != 0 && o->gemv_waves != 4 && o->gemv_waves != 8 && o->gemv_waves != 16)
    return false;
  out.kernel = o->kernel;
  out.gemv_split = o->gemv_split;
  out.gemv_waves = o->gemv_waves;
  out.m1_prep = o->m1_prep != 0;
  out.gemm_split = o->gemm_split;
  return true;
}

// The kernel a call runs.
int kernel_for(int64_t M, const msq::Options& o) {
  if (o.kernel != MSQ_KERNEL_AUTO) return o.kernel;
  return M <= MSQ_AUTO_GEMV_MAX_M ? MSQ_KERNEL_GEMV : MSQ_KERNEL_GEMM;
}

size_t workspace_for(int64_t M, int64_t N, int64_t K, const msq::Options& o) {
  if (M <= 0) return 0;
  if (kernel_for(M, o) == MSQ_KERNEL_GEMV)
    return M <= MSQ_GEMV_MAX_M ? msq::plan_gemv(M, N, K, o).workspace : 0;
  return msq::gemm_workspace_bytes(M, N, K, o);
}

msq_status gemm_impl(const uint16_t* x_bf16, int64_t M, const msq_weight* w, float* y,
                     void* workspace, size_t workspace_bytes, const msq::Options& o,
                     hipStream_t stream) {
  msq_status st = weight_ptrs_ok(w);
  if (st != MSQ_OK) return st;
  if (M < 0) return MSQ_ERR_SHAPE;
  if (M == 0) return MSQ_OK;
  if (M > (int64_t)0x7FFFFFFF / 2) return MSQ_ERR_SHAPE;
  if (!x_bf16 || !y || !aligned(x_bf16, 16) || !aligned(y, 4)) return MSQ_ERR_INVALID_ARG;
  const int kernel = kernel_for(M, o);
  if (kernel == MSQ_KERNEL_GEMV && M > MSQ_GEMV_MAX_M) return MSQ_ERR_UNSUPPORTED;
  const size_t need = workspace_for(M, w->N, w->K, o);
  if (need > 0 && (!workspace || !aligned(workspace, 256))) return MSQ_ERR_INVALID_ARG;
  if (workspace_bytes < need) return MSQ_ERR_BUFFER_TOO_SMALL;
  const msq::WeightView v = view_of(w);
  hipError_t e;
  if (kernel == MSQ_KERNEL_GEMV) {
    const msq::GemvPlan p = msq::plan_gemv(M, w->N, w->K, o);
    e = msq::launch_gemv(x_bf16, M, v, y, workspace, p, stream);
    // the decode kernel leaves 16-bit blocks to one more pass
    if (e == hipSuccess && w->tile16_blocks > 0)
      e = msq::launch_tile16(x_bf16, msq::gemv_reordered_x(workspace, p, M, w->N), M, v, y, stream);
  } else {
    e = msq::launch_gemm(x_bf16, M, v, y, workspace, o, stream);
  }
  return e == hipSuccess ? MSQ_OK : MSQ_ERR_HIP;
}

size_t group_workspace_impl(int64_t M, const msq_weight* const* w, int count, const msq::Options& o) {
  if (!w || count < 1 || count > MSQ_GROUP_MAX || M <= 0) return 0;
  msq::WeightView v[MSQ_GROUP_MAX];
  for (int i = 0; i < count; ++i) {
    if (!w[i] || check_shape(w[i]->N, w[i]->K) != MSQ_OK) return 0;
    v[i] = view_of(w[i]);
  }
  // every matrix keeps its own workspace (one launch for all, or split-K
  // single calls)
  if (M == 1) return msq::gemv_group_workspace_m1(v, count, o);
  if (M > MSQ_AUTO_GEMV_MAX_M) return msq::gemm_group_workspace_bytes(M, v, count, o);
  return msq::gemv_group_workspace_small(M, v, count, o);
}

msq_status group_impl(const uint16_t* const* x_bf16, int64_t M, const msq_weight* const* w,
                      float* const* y, int count, void* workspace, size_t workspace_bytes,
                      const msq::Options& o, hipStream_t stream) {
  static_assert(MSQ_GROUP_MAX == msq::kGemvGroupMax, "group size of the header and the kernels");
  static_assert(MSQ_AUTO_GEMV_MAX_M == msq::kGemvGroupMaxSmallM,
                "grouped decode covers every M the automatic choice sends to the decode kernel");
  if (!x_bf16 || !w || !y || count < 1 || count > MSQ_GROUP_MAX) return MSQ_ERR_INVALID_ARG;
  if (o.kernel != MSQ_KERNEL_AUTO) return MSQ_ERR_INVALID_ARG;
  for (int i = 0; i < count; ++i) {
    const msq_status st = weight_ptrs_ok(w[i]);
    if (st != MSQ_OK) return st;
    if (!x_bf16[i] || !y[i] || !aligned(x_bf16[i], 16) || !aligned(y[i], 4))
      return MSQ_ERR_INVALID_ARG;
  }
  if (M < 0) return MSQ_ERR_SHAPE;
  if (M == 0) return MSQ_OK;
  if (M > (int64_t)0x7FFFFFFF / 2) return MSQ_ERR_SHAPE;
  const size_t need = group_workspace_impl(M, w, count, o);
  if (need > 0 && (!workspace || !aligned(workspace, 256))) return MSQ_ERR_INVALID_ARG;
  if (workspace_bytes < need) return MSQ_ERR_BUFFER_TOO_SMALL;
  msq::WeightView v[MSQ_GROUP_MAX];
  for (int i = 0; i < count; ++i) v[i] = view_of(w[i]);
  if (M != 1 && M <= MSQ_AUTO_GEMV_MAX_M)
    return msq::launch_gemv_group_small(x_bf16, M, v, y, count, workspace, o, stream) == hipSuccess
               ? MSQ_OK
               : MSQ_ERR_HIP;
  if (M > 1)  // the prefill GEMM multiplies 16-bit blocks itself
    return msq::launch_gemm_group(x_bf16, M, v, y, count, workspace, o, stream) == hipSuccess
               ? MSQ_OK
               : MSQ_ERR_HIP;
  hipError_t e = msq::launch_gemv_group_m1(x_bf16, v, y, count, workspace, o, stream);
  for (int i = 0; i < count && e == hipSuccess; ++i)
    if (w[i]->tile16_blocks > 0) e = msq::launch_tile16(x_bf16[i], nullptr, 1, v[i], y[i], stream);
  return e == hipSuccess ? MSQ_OK : MSQ_ERR_HIP;
}

// ---- scratch for msq_gemm_noalloc ---------------------------------------------------------
// The workspace of msq_gemm_noalloc: a file-scope device array, one copy per
// GPU the library runs on, held until the process ends.  In host code its
// name is only a stand-in: kernels get the device address that
// hipGetSymbolAddress returns, looked up once per device with that device
// current and kept in scratch_ptr.
static __device__ __align__(256) uint8_t scratch[MSQ_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void* scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array, or nullptr.
void* device_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    scratch_ptr[dev] = p;
  }
  return scratch_ptr[dev];
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
  if (w->code_bytes < 0) return MSQ_ERR_INVALID_ARG;
  // The descriptor is trusted (its bits and permutations passed msq_plan):
  // nothing is read back, so the call stays asynchronous.  The kernels clamp
  // every index and skip blocks that would end past code_bytes.
  const int64_t N = w->N, K = w->K;
  const int64_t nblk = (N / kBlockRows) * (K / kBlockCols);
  if (hipError_t e = msq::launch_block_offsets(w->bits, nblk, w->block_offset, stream); e != hipSuccess)
    return MSQ_ERR_HIP;
  if (hipError_t e = msq::launch_pack(W_bf16, N, K, w->bits, w->perm_row, w->perm_col,
                                      w->block_offset, w->codes, w->code_bytes, w->scale, w->zero,
                                      stream);
      e != hipSuccess)
    return MSQ_ERR_HIP;
  return MSQ_OK;
}

size_t msq_gemm_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (check_shape(N, K) != MSQ_OK || M <= 0) return 0;
  // enough for either kernel, so msq_gemm_ex with only a kernel choice fits too
  msq::Options o;
  o.kernel = MSQ_KERNEL_GEMV;
  const size_t a = M <= MSQ_GEMV_MAX_M ? workspace_for(M, N, K, o) : 0;
  o.kernel = MSQ_KERNEL_GEMM;
  const size_t b = workspace_for(M, N, K, o);
  return a > b ? a : b;
}

size_t msq_gemm_workspace_bytes_ex(int64_t M, int64_t N, int64_t K, const msq_options* opt) {
  msq::Options o;
  if (!options_of(opt, o) || check_shape(N, K) != MSQ_OK || M <= 0) return 0;
  if (!opt) return msq_gemm_workspace_bytes(M, N, K);
  return workspace_for(M, N, K, o);
}

msq_status msq_gemm_ex(const uint16_t* x_bf16, int64_t M, const msq_weight* w, float* y,
                       void* workspace, size_t workspace_bytes, const msq_options* opt,
                       hipStream_t stream) {
  msq::Options o;
  if (!options_of(opt, o)) return MSQ_ERR_INVALID_ARG;
  return gemm_impl(x_bf16, M, w, y, workspace, workspace_bytes, o, stream);
}

msq_status msq_gemm(const uint16_t* x_bf16, int64_t M, const msq_weight* w, float* y,
                    void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return gemm_impl(x_bf16, M, w, y, workspace, workspace_bytes, msq::Options{}, stream);
}

size_t msq_gemm_group_workspace_bytes(int64_t M, const msq_weight* const* w, int count) {
  return group_workspace_impl(M, w, count, msq::Options{});
}

size_t msq_gemm_group_workspace_bytes_ex(int64_t M, const msq_weight* const* w, int count,
                                         const msq_options* opt) {
  msq::Options o;
  if (!options_of(opt, o) || o.kernel != MSQ_KERNEL_AUTO) return 0;
  return group_workspace_impl(M, w, count, o);
}

msq_status msq_gemm_group(const uint16_t* const* x_bf16, int64_t M, const msq_weight* const* w,
                          float* const* y, int count, void* workspace, size_t workspace_bytes,
                          hipStream_t stream) {
  return group_impl(x_bf16, M, w, y, count, workspace, workspace_bytes, msq::Options{}, stream);
}

msq_status msq_gemm_group_ex(const uint16_t* const* x_bf16, int64_t M, const msq_weight* const* w,
                             float* const* y, int count, void* workspace, size_t workspace_bytes,
                             const msq_options* opt, hipStream_t stream) {
  msq::Options o;
  if (!options_of(opt, o)) return MSQ_ERR_INVALID_ARG;
  return group_impl(x_bf16, M, w, y, count, workspace, workspace_bytes, o, stream);
}

msq_status msq_gemm_noalloc(const uint16_t* x_bf16, int64_t M, const msq_weight* w, float* y,
                            hipStream_t stream) {
  msq_status st = weight_ptrs_ok(w);
  if (st != MSQ_OK) return st;
  if (M < 0) return MSQ_ERR_SHAPE;
  if (M == 0) return MSQ_OK;
  if (M > (int64_t)0x7FFFFFFF / 2) return MSQ_ERR_SHAPE;
  const msq::Options o{};
  if (workspace_for(M, w->N, w->K, o) > (size_t)MSQ_NOALLOC_SCRATCH_BYTES)
    return MSQ_ERR_BUFFER_TOO_SMALL;
  // Every buffer the kernels need at zero is cleared by the kernels
  // themselves each call (the M == 1 split counters by the activation-prep
  // launch); everything else they read is written earlier in the same call.
  void* ws = device_scratch();
  if (!ws) return MSQ_ERR_HIP;
  return gemm_impl(x_bf16, M, w, y, ws, (size_t)MSQ_NOALLOC_SCRATCH_BYTES, o, stream);
}

const char* msq_status_string(int s) {
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
