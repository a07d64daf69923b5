// fa2_merge.hip — merge of partial attention results by their logsumexp (gfx950), and its C
// ABI (declared in include/fa2.h).
//
// Attention over a key set that is split into parts (key/value chunks on one GPU, or shards
// of the key sequence on several) is recovered exactly from each part's normalised output
// O_s and logsumexp LSE_s:
//     LSE = log sum_s exp(LSE_s),    O = sum_s exp(LSE_s - LSE) O_s
// This is the same rescaling the online softmax applies between key blocks, applied once
// across parts ("FlashAttention" on llm-infra-atlas: section 5 describes context parallelism
// as one FlashAttention call per key shard with the right mask; the reading table of its
// section 0 lists sparse variants that combine two variable-length calls by mixing their
// LSEs). A part in which a row has no allowed key carries O_s = 0 and LSE_s = -inf and gets
// weight zero; a row with no allowed key in any part gets O = 0 and LSE = -inf.
//
// The kernel is bound by HBM bandwidth (it reads every part once and writes the result once):
// a row of D bf16 is handled by D/8 lanes, 16 bytes each, so every part's row is one
// contiguous, fully used read. Weights are computed in fp32 with the base-2 exponential.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "fa2.h"
#include "fa2_dev.h"

namespace {

// D: 64, 128 or 256, at least the tensors' head dimension dg (a multiple of 8); lanes past
// dg / 8 only compute the row's weights.
template <int D>
__global__ __launch_bounds__(256) void fa2_lse_merge_kernel(const uint16_t* __restrict__ o_parts,
                                                            const float* __restrict__ lse_parts,
                                                            int num_parts, long long rows, int dg,
                                                            uint16_t* __restrict__ o,
                                                            float* __restrict__ lse) {
  constexpr int LPR = D / 8;          // lanes per row
  constexpr int RPB = 256 / LPR;      // rows per workgroup
  const long long row = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  if (row >= rows) return;
  const bool has_cols = part * 8 < dg;

  float m = -INFINITY;
  for (int s = 0; s < num_parts; ++s) m = fmaxf(m, lse_parts[(size_t)s * rows + row]);

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float z = 0.f;
  if (m != -INFINITY) {
    for (int s = 0; s < num_parts; ++s) {
      const float w = __builtin_amdgcn_exp2f((lse_parts[(size_t)s * rows + row] - m) * kLog2e);
      u32x4 t = {0u, 0u, 0u, 0u};
      if (has_cols) t = *(const u32x4*)(o_parts + ((size_t)s * rows + row) * dg + part * 8);
      z += w;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += w * __uint_as_float(t[e] << 16);
        acc[2 * e + 1] += w * __uint_as_float(t[e] & 0xffff0000u);
      }
    }
  }
  const float inv = z > 0.f ? 1.f / z : 0.f;
  const u32x4 out = {pack_bf16x2(acc[0] * inv, acc[1] * inv), pack_bf16x2(acc[2] * inv, acc[3] * inv),
                     pack_bf16x2(acc[4] * inv, acc[5] * inv), pack_bf16x2(acc[6] * inv, acc[7] * inv)};
  if (has_cols) *(u32x4*)(o + (size_t)row * dg + part * 8) = out;
  if (part == 0) lse[row] = z > 0.f ? m + __builtin_amdgcn_logf(z) * kLn2 : -INFINITY;
}

// Few rows against many parts (split-KV for a handful of query rows): one workgroup per row,
// the parts spread over 256 / (D/8) lane groups so that the loads of every part are in flight
// at once instead of one part after another. Each group folds its parts into a running
// (max, sum, weighted O) with the same rescaling as the merge formula, and the groups are
// combined through LDS.
template <int D>
__global__ __launch_bounds__(256) void fa2_lse_merge_rows_kernel(const uint16_t* __restrict__ o_parts,
                                                                 const float* __restrict__ lse_parts,
                                                                 int num_parts, long long rows, int dg,
                                                                 uint16_t* __restrict__ o,
                                                                 float* __restrict__ lse) {
  constexpr int LPR = D / 8;          // lanes per part row
  constexpr int PG = 256 / LPR;       // part groups
  __shared__ float red[PG][2 + D];
  const long long row = blockIdx.x;
  const int pg = threadIdx.x / LPR;
  const int ch = threadIdx.x % LPR;
  const bool has_cols = ch * 8 < dg;

  float m = -INFINITY, z = 0.f;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int s = pg; s < num_parts; s += PG) {
    const float ls = lse_parts[(size_t)s * rows + row];
    u32x4 t = {0u, 0u, 0u, 0u};
    if (has_cols) t = *(const u32x4*)(o_parts + ((size_t)s * rows + row) * dg + ch * 8);
    if (ls == -INFINITY) continue;   // a part without keys for this row: weight zero
    const float M = fmaxf(m, ls);
    const float a = __builtin_amdgcn_exp2f((m - M) * kLog2e);   // 0 while m = -inf
    const float w = __builtin_amdgcn_exp2f((ls - M) * kLog2e);
    z = z * a + w;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] = acc[2 * e] * a + w * __uint_as_float(t[e] << 16);
      acc[2 * e + 1] = acc[2 * e + 1] * a + w * __uint_as_float(t[e] & 0xffff0000u);
    }
    m = M;
  }
  if (ch == 0) {
    red[pg][0] = m;
    red[pg][1] = z;
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[pg][2 + ch * 8 + e] = acc[e];
  __syncthreads();
  if (pg != 0) return;
  float M = -INFINITY;
  for (int g = 0; g < PG; ++g) M = fmaxf(M, red[g][0]);
  float Z = 0.f;
  float out[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
    for (int g = 0; g < PG; ++g) {
      const float w = __builtin_amdgcn_exp2f((red[g][0] - M) * kLog2e);   // 0 for empty groups
      Z += w * red[g][1];
#pragma unroll
      for (int e = 0; e < 8; ++e) out[e] += w * red[g][2 + ch * 8 + e];
    }
  }
  const float inv = Z > 0.f ? 1.f / Z : 0.f;
  const u32x4 w = {pack_bf16x2(out[0] * inv, out[1] * inv), pack_bf16x2(out[2] * inv, out[3] * inv),
                   pack_bf16x2(out[4] * inv, out[5] * inv), pack_bf16x2(out[6] * inv, out[7] * inv)};
  if (has_cols) *(u32x4*)(o + (size_t)row * dg + ch * 8) = w;
  if (ch == 0) lse[row] = Z > 0.f ? M + __builtin_amdgcn_logf(Z) * kLn2 : -INFINITY;
}

// Rows up to which a merge of 4 or more parts takes one workgroup per row.
constexpr long long kMergeRowsPerRowKernel = 4096;

bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

}  // namespace

extern "C" {

int fa2_lse_merge(const void* o_parts, const float* lse_parts, int num_parts, long long rows,
                  int d, void* o, float* lse, void* stream) {
  if (num_parts <= 0 || rows < 0) return FA2_ERR_BAD_SHAPE;
  if (d < 8 || d > 256 || d % 8 != 0) return FA2_ERR_UNSUPPORTED_HEADDIM;
  if (rows == 0) return FA2_OK;
  if (!o_parts || !lse_parts || !o || !lse) return FA2_ERR_NULL_PTR;
  if (!aligned16(o_parts) || !aligned16(o) || ((uintptr_t)lse_parts & 3) || ((uintptr_t)lse & 3))
    return FA2_ERR_MISALIGNED;
  const int dpad = d <= 64 ? 64 : d <= 128 ? 128 : 256;
  const int rpb = 256 / (dpad / 8);
  const long long blocks = (rows + rpb - 1) / rpb;
  if (blocks > 0x7fffffffLL || (long long)num_parts * rows > (1LL << 40)) return FA2_ERR_TOO_LARGE;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FA2_ERR_NO_DEVICE;
  // Few rows and several parts: one workgroup per row with the parts read in parallel (the
  // row-per-lane-group kernel would walk the parts one after another in a handful of
  // workgroups); otherwise rows are spread over lane groups.
  const bool per_row = num_parts >= 4 && rows <= kMergeRowsPerRowKernel;
  const void* fn;
  if (per_row)
    fn = dpad == 64    ? (const void*)&fa2_lse_merge_rows_kernel<64>
         : dpad == 128 ? (const void*)&fa2_lse_merge_rows_kernel<128>
                       : (const void*)&fa2_lse_merge_rows_kernel<256>;
  else
    fn = dpad == 64    ? (const void*)&fa2_lse_merge_kernel<64>
         : dpad == 128 ? (const void*)&fa2_lse_merge_kernel<128>
                       : (const void*)&fa2_lse_merge_kernel<256>;
  const uint16_t* op = (const uint16_t*)o_parts;
  uint16_t* oo = (uint16_t*)o;
  void* args[] = {&op, &lse_parts, &num_parts, &rows, &d, &oo, &lse};
  hipError_t e = hipLaunchKernel(fn, dim3((unsigned)(per_row ? rows : blocks)), dim3(256), args, 0,
                                 (hipStream_t)stream);
  return e == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}

}  // extern "C"
