// Internal declarations of the msq library: launch helpers implemented in the
// .hip translation units and called by the C-ABI layer (msq_host.cpp).
// Nothing here is part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msq {

constexpr int kBlockRows = 64;    // rows of W per block (along N)
constexpr int kBlockCols = 128;   // columns of W per block (along K) = one RTN group
constexpr uint32_t kNoBlock = 0xFFFFFFFFu;

// Plain-old-data view of a packed weight passed to kernels.
struct WeightView {
  int64_t N, K;
  int NBr, NBc;                // N / 64, K / 128
  const uint8_t* bits;         // [NBr][NBc]
  const int32_t* perm_row;     // [N]
  const int32_t* perm_col;     // [K]
  const uint32_t* block_offset;// [NBr][NBc] KiB
  const uint8_t* codes;
  const float* scale;          // [NBr][NBc][64]
  const uint8_t* zero;         // [NBr][NBc][64]
  int has16;                   // the bit map holds 16-bit (passthrough) blocks
};

// Launch choices (the public msq_options, validated by the C-ABI layer).
struct Options {
  int kernel = 0;      // 0 auto, 1 GEMV, 2 GEMM
  int gemv_split = 0;  // 0 automatic
  int gemv_waves = 0;  // 0 automatic, else 4, 8, 16 (M == 1)
  int m1_prep = 0;     // nonzero: M == 1 always reorders x in the prep launch
  int gemm_split = 0;  // 0 automatic
};

// ---- pack (msq_pack.hip)
hipError_t launch_block_offsets(const uint8_t* bits, int64_t nblocks, uint32_t* offsets,
                                hipStream_t stream);
hipError_t launch_pack(const uint16_t* W, int64_t N, int64_t K, const uint8_t* bits,
                       const int32_t* perm_row, const int32_t* perm_col,
                       const uint32_t* offsets, uint8_t* codes, int64_t code_bytes, float* scale,
                       uint8_t* zero, hipStream_t stream);

// ---- decode GEMV, M <= 64 (msq_gemv.hip)
struct GemvPlan {
  int split;        // K-splits across workgroups
  int kr;           // block columns per split (<= 64)
  int nw;           // wavefronts per workgroup
  int gather;       // M == 1: the workgroups reorder x themselves (no prep launch)
  int halves;       // M == 1: two workgroups per block row of 32 rows each (gather, split 1)
  size_t lds_bytes; // dynamic LDS per workgroup
  size_t workspace; // bytes: fp32 partials (split > 1), then M == 1 prep or M > 1 gather buffers
};
// group_rows > 0: the plan of one matrix of a grouped launch whose matrices
// have group_rows output rows in total (the K split then fills the GPU with
// the whole group's workgroups).
GemvPlan plan_gemv(int64_t M, int64_t N, int64_t K, const Options& opt,
                   int64_t group_rows = 0);
hipError_t launch_gemv(const uint16_t* x, int64_t M, const WeightView& w, float* y,
                       void* workspace, const GemvPlan& plan, hipStream_t stream);

// y[m][perm_row[n]] += the exact bf16 product of the 16-bit (passthrough)
// blocks of every block row: one launch after the decode kernel (the
// prefill GEMM multiplies 16-bit blocks itself).  xr:
// the reordered x [M][K] those kernels left in the workspace, or null.
hipError_t launch_tile16(const uint16_t* x, const uint16_t* xr, int64_t M, const WeightView& w,
                         float* y, hipStream_t stream);
// The reordered x [M][K] that launch_gemv (M > 1) leaves in its workspace.
const uint16_t* gemv_reordered_x(void* workspace, const GemvPlan& p, int64_t M, int64_t N);

// Grouped M == 1 decode of count (1 .. 8) matrices in one decode launch (and
// one prep launch for those with several K ranges); the workspace holds each
// matrix's single-call workspace in turn.
constexpr int kGemvGroupMax = 8;
size_t gemv_group_workspace_m1(const WeightView* w, int count, const Options& opt);
hipError_t launch_gemv_group_m1(const uint16_t* const* x, const WeightView* w, float* const* y,
                                int count, void* workspace, const Options& opt,
                                hipStream_t stream);
// Grouped decode at 2 <= M <= kGemvGroupMaxSmallM (the automatic choice's
// limit; one or two m tiles): one gather launch, one decode launch over
// all matrices (each planned with the group's rows), one reduction launch for
// the matrices with several K ranges, then the 16-bit pass of each matrix
// that has 16-bit blocks; the workspace holds each matrix's workspace in turn.
constexpr int kGemvGroupMaxSmallM = 32;
size_t gemv_group_workspace_small(int64_t M, const WeightView* w, int count, const Options& opt);
hipError_t launch_gemv_group_small(const uint16_t* const* x, int64_t M, const WeightView* w,
                                   float* const* y, int count, void* workspace, const Options& opt,
                                   hipStream_t stream);

// ---- activation gather for M > 1 (msq_gemm.hip): x_r[m][j] = x[m][perm_col[j]]
// and the group sums of x_r split into three bf16 terms S0 + S1 + S2 (exact
// fp32), [3][M][Gp] with Gp = the group count rounded up to 32.  It writes
// into gather_workspace_bytes(M, K) bytes at ws: x_r first, the sums 256-byte
// aligned after it, then (on request) the fp32 sums.
__host__ __device__ constexpr int64_t padded_groups(int64_t G) { return (G + 31) & ~(int64_t)31; }
// Rows of the fp32 group sums: M rounded up to 16.
__host__ __device__ constexpr int64_t gather_mpad(int64_t M) { return (M + 15) & ~(int64_t)15; }
size_t gather_workspace_bytes(int64_t M, int64_t K);
// sums_f32: also write the group sums in fp32, [padded groups][gather_mpad(M)]
// (rows past M left as they are), at gather_sums_f32(ws, M, K).  The
// gather's workgroups also zero counters[0 .. ncounters - 1] (the K-split
// counters of the decode launch that follows it; nullptr and 0 for none).
hipError_t launch_gather_x(const uint16_t* x, int64_t M, const WeightView& w, void* ws,
                           hipStream_t stream, bool sums_f32, uint32_t* counters,
                           int ncounters);
float* gather_sums_f32(void* ws, int64_t M, int64_t K);
// The gather of launch_gather_x (sums_f32 on) for count (1 .. 8) matrices at
// one M in one launch; ws[i] is matrix i's gather workspace, counters[i] and
// ncounters[i] its decode's K-split counters.
hipError_t launch_gather_x_group(const uint16_t* const* x, int64_t M, const WeightView* w,
                                 void* const* ws, uint32_t* const* counters,
                                 const int* ncounters, int count, hipStream_t stream);

// ---- K-split reduction (msq_gemv.hip): y[m][perm_row[n]] = sum over splits,
// in split order, of part[sp][m][n].
hipError_t launch_split_reduce(const float* part, int split, int64_t M, int64_t N,
                               const int32_t* perm_row, float* y, hipStream_t stream);

// ---- prefill GEMM, any M (msq_gemm.hip).  Workspace: the gather buffers,
// then (when the call splits K to fill the GPU) fp32 partials.
size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, const Options& opt);
hipError_t launch_gemm(const uint16_t* x, int64_t M, const WeightView& w, float* y,
                       void* workspace, const Options& opt, hipStream_t stream);
// Grouped prefill of count (1 .. 8) matrices at one M: one gather and one GEMM
// launch; the workspace holds each matrix's single-call workspace in turn.
size_t gemm_group_workspace_bytes(int64_t M, const WeightView* w, int count, const Options& opt);
hipError_t launch_gemm_group(const uint16_t* const* x, int64_t M, const WeightView* w,
                             float* const* y, int count, void* workspace, const Options& opt,
                             hipStream_t stream);

}  // namespace msq
