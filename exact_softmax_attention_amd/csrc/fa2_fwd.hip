// fa2_fwd.hip — gfx950 (CDNA4) forward kernels for exact softmax attention, and the C ABI
// declared in include/fa2.h.
//
// Page abbreviations used below:
//   [CHL] "FlashAttention 2: Faster Attention with Better Parallelism and Work Partitioning",
//         reading notes at papers.chlience.com
//   [LAN] "Flash Attention 2 (FA2)", languisher.top
//   [ATL] "FlashAttention", llm-infra-atlas
//   [PGU] "FlashAttention-2: Faster Attention with Better Parallelism and Work Partitioning",
//         paper-graph-ui summary
//
// One workgroup owns a block of query rows of one (batch, head) or (sequence, head) pair
// and walks the key/value tiles of BC keys in order ([CHL] 5.1, 5.4: query row blocks are
// the outer, parallel loop; key/value blocks the inner, sequential one). Each 64-lane wave
// owns 32 whole query rows, so no statistic is ever shared between waves ([CHL] 5.5
// split-Q; [PGU] 3.4 "warp-level work partitioning"). Per tile and wave:
//
//   S^T  = K_j Q_i^T          bf16 MFMA 32x32x16, fp32 accumulate      (a4)
//   mask                      only on diagonal / ragged tiles            (a5)
//   m'   = max(m, rowmax S·c); P~ = exp2(S·c - m'); l = 2^(m-m') l + rowsum P~   (a6)
//   O~^T = 2^(m-m') O~^T + V_j^T P~^T   bf16 MFMA, fp32 accumulate      (a7)
//
// and after the last tile O = O~ / l, LSE = (m + log2 l)·ln2 ([CHL] 5.2; [PGU] 3.4
// "Algorithm 1 Walkthrough"; the rescale multiplies by 2^(m-m') <= 1 as in the erratum of
// [LAN] "减少非矩阵乘法运算"). c = scale·log2(e) folds the softmax scale into the base-2
// exponential the hardware provides (v_exp_f32 computes 2^x); [ATL] 2 notes the upstream
// rescale also uses exp2. The reference max m may lag the true running max (kLazy,
// kOptimistic below); the result is the same because m cancels in O~/l and in m + log2 l.
//
// Why S^T and not S: a 32x32 MFMA result gives each lane one column and 16 rows. Computing
// S^T = K Q^T puts one query per lane column, so a lane holds 16 keys of a single query per
// 32-key block: the row max and row sum are in-lane, plus one exchange between the two
// 32-lane halves (v_permlane32_swap). The same lane layout is exactly the B operand the PV
// product needs (O^T = V^T P^T, one query per lane column, 8 contraction positions per lane),
// so P~ never leaves registers. For contraction step c, operand position 8h + 4t + e (h =
// lane half, t = 0/1, e = 0..3) carries key 16c + 8t + 4h + e on both sides; the V^T operand
// is gathered from the row-major V tile in LDS with two LDS transpose reads
// (ds_read_b64_tr_b16) in exactly that key order.
//
// K and V tiles move from global memory straight into LDS (global_load_lds_dwordx4), with
// their 16-byte chunks XOR-swizzled by row so that every operand read is bank-conflict free.
//
// MFMA lane layouts used (v_mfma_f32_32x32x16_bf16, wave64, lane l, element e):
//   A[m][k]: m = l % 32, k = 8*(l / 32) + e          (8 bf16 per lane)
//   B[k][n]: n = l % 32, k = 8*(l / 32) + e          (8 bf16 per lane)
//   C[m][n]: n = l % 32, m = 8*(r / 4) + 4*(l / 32) + r % 4, r = 0..15   (16 fp32 per lane)
// ds_read_b64_tr_b16 (per 16-lane group, lane j of the group receives element j % 4 of the
// 8-byte rows addressed by lanes 4e + (j % 16) / 4, e = 0..3).

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <algorithm>
#include <mutex>

#include "fa2.h"
#include "fa2_dev.h"

namespace {

// Kernel arguments (passed by value).
struct Params {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;
  const int* cu_seqlens;  // varlen only
  int nb;                 // batch size, or number of sequences (varlen)
  int dg;                 // head dimension of the tensors (a multiple of 8, <= D; the kernel's
                          // D is the next of 64 / 128 / 256 and the extra columns are zero
                          // in Q and never written in O)
  int H;                  // query heads
  int Hkv;                // key/value heads (H for MHA)
  int g;                  // query heads per key/value head, H / Hkv
  int N;                  // query rows per sequence, or max_seqlen (varlen)
  int Nk;                 // keys per sequence (fixed length; varlen uses the sequence length)
  int diag;               // causal: query i may attend key j iff j <= i + diag
  int split_len;          // keys per split (split-KV: blockIdx.y selects the split); Nk if none
  long long part_rows;    // split s writes O/LSE rows s * part_rows + ... (0 if not split)
  int T;                  // tokens per head plane: N, or total_tokens (varlen)
  int tr;                 // row blocks per (batch|sequence, head)
  int heads_per_xcd;      // > 0: XCD-aware workgroup order (nb*H divisible by 8)
  float c;                // |scale| * log2(e), at least 1e-30
  uint32_t qflip;         // 0x80008000 negates Q (scale < 0), else 0
};

// Compile-time tile geometry. NW waves of 32 query rows share each K/V tile (NW = 8 puts
// one 256-row workgroup on a CU, two waves per SIMD, and halves the K/V staging per query
// row against NW = 4). K and V tiles are BC rows of D bf16 (row pitch 2*D bytes, no
// padding), stored in LDS with their 16-byte chunks permuted by an XOR of low row bits so
// that the MFMA operand reads below hit distinct banks.
template <int D, int BC, int NW = 4>
struct Tile {
  static constexpr int WAVES = NW;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BR = 32 * WAVES;             // query rows per workgroup
  static constexpr int ROWB = 2 * D;                // bytes per K or V row
  static constexpr int TILEB = BC * ROWB;           // bytes per K (or V) tile
  static constexpr int STAGEB = 2 * TILEB;          // K tile then V tile
  static constexpr int LDS_BYTES = 2 * STAGEB;      // double buffered
  static constexpr int DMA_PER_WAVE = TILEB / 1024 / WAVES;  // 1 KB direct loads per wave
  static constexpr int NKB = BC / 32;               // 32-key blocks per tile
  static constexpr int NKC = D / 16;                // 16-wide contraction steps of QK^T
  static constexpr int NDB = D / 32;                // 32-wide d blocks of O^T
  static constexpr int NPC = BC / 16;               // 16-key contraction steps of PV
  static_assert(D == 64 || D == 128 || D == 256, "head dim");
  static_assert(BC % 32 == 0 && TILEB % (1024 * WAVES) == 0, "tile shape");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");

  // Swizzle of K rows: lanes reading 16 consecutive rows at one logical chunk land in 16
  // distinct 16-byte bank groups.
  __device__ static int kswz(int row) { return D >= 128 ? (row & 15) : ((row >> 1) & 7); }
  // Swizzle of V rows: a transposed read touches 4 consecutive rows x 2..4 chunks.
  __device__ static int vswz(int row) { return D >= 128 ? ((row & 3) << 2) : (((row >> 1) & 1) << 2); }
};

// Workgroup id -> (batch|sequence * H + head, row block). With the XCD-aware order,
// workgroup id goes to XCD id % 8 (round-robin dispatch), and each XCD is given a
// contiguous set of heads so the K/V of a head stay in one XCD's L2. Causal launches visit
// row blocks heaviest first (largest i has the most key tiles).
template <bool CAUSAL>
__device__ __forceinline__ void decode_block(const Params& p, int id, int& bh, int& i) {
  if (p.heads_per_xcd > 0) {
    const int x = id & 7, slot = id >> 3, hpx = p.heads_per_xcd;
    int hl;
    if (CAUSAL) {
      i = p.tr - 1 - slot / hpx;
      hl = slot - (slot / hpx) * hpx;
    } else {
      hl = slot / p.tr;
      i = slot - hl * p.tr;
    }
    bh = x * hpx + hl;
  } else {
    const int nbh = p.nb * p.H;
    i = p.tr - 1 - id / nbh;
    bh = id - (id / nbh) * nbh;
  }
}

// Softmax bookkeeping modes. All three give the same O = O~ / l and LSE = m + log2 l up to
// rounding, because the reference value m cancels between numerator and denominator; they
// differ in how often the row max is computed and the accumulator rescaled.
//   kExact:      the pages' recurrence: m = max(m, rowmax) every tile, rescale when it grows.
//   kLazy:       rowmax every tile, but m only moves when a tile exceeds it by 2^kLazyTau.
//   kOptimistic: P~ is formed with the current m first; only when a lane's tile sum exceeds
//                2^kOptTau (or on the row's first tile) is the true row max taken, the
//                state rescaled and P~ formed again. m only grows and never passes the
//                true running max, so no entry underflows earlier than with kExact, and
//                every P~ entry is at most 2^kOptTau. The bound only has to keep the fp32
//                sums far from overflow (O~ stays below N * 2^kOptTau * max|V|); bf16 and
//                fp32 rounding are relative, so the size of the entries does not matter.
enum { kExact = 0, kLazy = 1, kOptimistic = 2 };
constexpr float kLazyTau = 8.0f;
constexpr float kOptTau = 16.0f;
constexpr float kOptLimit = (float)(1u << (int)kOptTau);   // 2^kOptTau

// A wave's Q^T fragments for its 32 query rows (lane: row qrow, 8 columns per step from
// 16kc + 8hl), loaded without branches so that every load issues at once: a branch around a
// load makes the compiler merge the loaded and the default value in a way that waits for
// that load in the middle of the sequence, one full memory latency at every workgroup's
// start. A row past the end of the sequence reads row seq_len - 1 instead: its column of S^T
// concerns no other row, and its O and LSE are never written. Columns past dg (a padded head
// dimension) are zeroed (col_mask), because K's padded columns repeat real ones.
template <int NKC>
__device__ __forceinline__ void load_q_fragments(bf16x8 (&qf)[NKC], const uint16_t* __restrict__ qh, int qrow,
                                                 int seq_len, int dg, int hl, uint32_t qflip) {
  const size_t base = (size_t)min(qrow, seq_len - 1) * (size_t)dg;
  u32x4 t[NKC];
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) {
    const int col = kc * 16 + hl * 8;
    t[kc] = *(const u32x4*)(qh + base + (col < dg ? col : 0));
  }
#pragma unroll
  for (int kc = 0; kc < NKC; ++kc) qf[kc] = as_bf16x8((t[kc] & col_mask(kc * 16 + hl * 8, dg)) ^ qflip);
}

// One row block (work item id): the whole forward for BR query rows of one (sequence, head).
// LA: how many operand fragments are read from LDS ahead of the MFMA that consumes them
// (0 leaves the order to the compiler's scheduler). RING: the K and V^T fragments of every
// tile are read from explicit register rings fenced by scheduling barriers. Called once per
// workgroup the scheduling-group hints already pipeline the 64-key tiles (RING = false);
// nested in the persistent kernel's loop over blocks they no longer hold (RING = true).
template <int D, int BC, bool CAUSAL, bool VARLEN, int MODE, int LA, int NW, bool RING>
__device__ __forceinline__ void fwd_block(const Params& p, int id) {
  using TL = Tile<D, BC, NW>;
  __shared__ __attribute__((aligned(1024))) unsigned char lds0[TL::STAGEB];
  __shared__ __attribute__((aligned(1024))) unsigned char lds1[TL::STAGEB];

  int tid = threadIdx.x;
  // In the persistent kernel this block is one iteration of a loop over blocks. An opaque
  // copy of the thread id keeps the compiler from hoisting the lane-derived offsets out of
  // that loop, where they would stay live across every block.
  if constexpr (RING) asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform per wave
  const int l32 = lane & 31;   // MFMA column (query) / A-row index
  const int hl = lane >> 5;    // which 32-lane half

  // ---- a1: work decode ----------------------------------------------------------------
  int bh, i;
  decode_block<CAUSAL>(p, id, bh, i);
  const int bi = bh / p.H;
  const int h = bh - bi * p.H;
  int seq_len, seq_k;   // query rows and keys of this sequence
  // Grouped/multi-query attention: query head h reads key/value head h / g, so the g query
  // heads of a group share one K/V plane without copies.
  const int hk = h / p.g;
  size_t row0;    // index of this sequence's first token in the Q/O/LSE [.., T, D] arrays
  size_t kvrow0;  // the same token in the K/V arrays
  if (VARLEN) {
    int a = p.cu_seqlens[bi];
    int e = p.cu_seqlens[bi + 1];
    a = min(max(a, 0), p.T);
    e = min(max(e, a), p.T);
    seq_len = e - a;
    seq_k = seq_len;
    row0 = (size_t)h * (size_t)p.T + (size_t)a;
    kvrow0 = (size_t)hk * (size_t)p.T + (size_t)a;
  } else {
    seq_len = p.N;
    seq_k = p.Nk;
    row0 = (size_t)bh * (size_t)p.N;
    kvrow0 = ((size_t)bi * (size_t)p.Hkv + (size_t)hk) * (size_t)p.Nk;
  }
  // Split-KV: split s of the launch owns keys [s*split_len, (s+1)*split_len) and writes its
  // partial O and LSE to part s of the output (rows offset by s*part_rows).
  const int ks0 = VARLEN ? 0 : (int)blockIdx.y * p.split_len;
  if (!VARLEN) {
    seq_k = max(min(p.split_len, seq_k - ks0), 0);
    kvrow0 += (size_t)ks0;
  }
  const int diag = p.diag - ks0;
  const size_t orow0 = row0 + (VARLEN ? 0 : (size_t)blockIdx.y * (size_t)p.part_rows);
  const int q0 = i * TL::BR;
  if (q0 >= seq_len) return;  // uniform over the workgroup (varlen rows past the end)

  const int dg = p.dg;            // row pitch of Q, K, V, O in elements
  const int growb = 2 * dg;       // ... in bytes
  const uint16_t* __restrict__ qh = p.q + row0 * dg;
  const unsigned char* kh = (const unsigned char*)(p.k + kvrow0 * dg);
  const unsigned char* vh = (const unsigned char*)(p.v + kvrow0 * dg);

  // Key tiles to visit: causal stops after the tile holding the last key this block's last
  // query may attend (none when the whole key range lies after it).
  const int kv_end = max(CAUSAL ? min(seq_k, q0 + TL::BR + diag) : seq_k, 0);
  const int nt = (kv_end + BC - 1) / BC;

  // ---- a2: this wave's 32 query rows as MFMA B fragments (Q^T), once -----------------
  const int qw0 = q0 + wave * 32;           // first query row of this wave
  const int qrow = qw0 + l32;               // the query this lane's column holds
  bf16x8 qf[TL::NKC];
  load_q_fragments<TL::NKC>(qf, qh, qrow, seq_len, dg, hl, p.qflip);

  // ---- a3: K/V staging: global -> LDS directly (1 KB per wave instruction) ------------
  // Instruction b of a tile writes LDS bytes [1024 b, 1024 b + 1024); lane l's 16 bytes land
  // at 1024 b + 16 l, i.e. row r = (1024 b + 16 l) / ROWB, physical chunk pch. The lane
  // therefore fetches the logical chunk pch ^ swz(r) of global row r.
  int drow[TL::DMA_PER_WAVE];         // tile row each direct load fills
  uint32_t koff[TL::DMA_PER_WAVE];    // byte offset inside the tile's global rows (K)
  uint32_t voff[TL::DMA_PER_WAVE];    // same for V
#pragma unroll
  for (int d = 0; d < TL::DMA_PER_WAVE; ++d) {
    const int b = wave * TL::DMA_PER_WAVE + d;
    const int o = b * 1024 + lane * 16;
    const int r = o / TL::ROWB;
    const int pch = (o % TL::ROWB) / 16;
    drow[d] = r;
    // Padded columns (logical chunk beyond dg) load a real chunk of the same row: finite, and
    // multiplied by Q's zero columns (K) or landing in unwritten O columns (V).
    koff[d] = r * growb + (((pch ^ TL::kswz(r)) % (dg / 8)) * 16);
    voff[d] = r * growb + (((pch ^ TL::vswz(r)) % (dg / 8)) * 16);
  }

  auto dma_tile = [&](int j, unsigned char* stage) {
    const int key0 = j * BC;
    const unsigned char* kt = kh + (size_t)key0 * growb;
    const unsigned char* vt = vh + (size_t)key0 * growb;
    const uint32_t ks_a = lds_addr(stage) + wave * TL::DMA_PER_WAVE * 1024;
    const uint32_t vs_a = lds_addr(stage + TL::TILEB) + wave * TL::DMA_PER_WAVE * 1024;
    if (key0 + BC <= seq_k) {
#pragma unroll
      for (int d = 0; d < TL::DMA_PER_WAVE; ++d) {
        dma16(kt, koff[d], ks_a + d * 1024);
        dma16(vt, voff[d], vs_a + d * 1024);
      }
    } else {
      // Ragged last tile: rows past the end re-read the last valid row, so every value in
      // LDS is finite (its probability is zero after the mask).
      const int last = seq_k - 1 - key0;
#pragma unroll
      for (int d = 0; d < TL::DMA_PER_WAVE; ++d) {
        const uint32_t back = (uint32_t)(drow[d] - min(drow[d], last)) * growb;
        dma16(kt, koff[d] - back, ks_a + d * 1024);
        dma16(vt, voff[d] - back, vs_a + d * 1024);
      }
    }
  };

  // Per-lane LDS read offsets (bytes inside a stage), precomputed once. The swizzles only
  // permute the low four bits of a row's 16-byte chunk index, so logical chunk c + 16 lies
  // exactly 256 bytes after chunk c: offsets are kept for the first 16 chunks of a row and
  // the rest reached through the instructions' immediate offset (at d = 256 this keeps 12
  // registers fewer; at d <= 128 every offset is within the first 16 chunks anyway).
  //  K (A operand of S^T): row kb*32 + l32, logical chunk 2*kc + hl.
  constexpr int NKA = TL::NKC < 8 ? TL::NKC : 8;
  int kaddr[NKA];
#pragma unroll
  for (int kc = 0; kc < NKA; ++kc)
    kaddr[kc] = l32 * TL::ROWB + (((2 * kc + hl) ^ TL::kswz(l32)) * 16);
  //  V^T (A operand of O^T) by two transposed 8-byte reads per fragment from row-major V:
  //  the lane supplies row 16c + 8t + 4hl + (lane%16)/4 and columns 32db + 16((lane/16)%2) +
  //  4(lane%4) .. +3, and receives keys 16c + 8t + 4hl + 0..3 of column d = 32db + l32.
  const int vr = 4 * hl + ((lane & 15) >> 2);
  constexpr int NVA = TL::NDB < 4 ? TL::NDB : 4;
  int vaddr[NVA];
#pragma unroll
  for (int db = 0; db < NVA; ++db) {
    const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    vaddr[db] = TL::TILEB + vr * TL::ROWB + (((col >> 3) ^ TL::vswz(vr)) * 16) + (col & 7) * 2;
  }

  // ---- running state (fp32, registers) -----------------------------------------------
  f32x16 oacc[TL::NDB];
#pragma unroll
  for (int db = 0; db < TL::NDB; ++db) oacc[db] = (f32x16){};
  float m_run = -INFINITY;  // reference max of S·c (base-2 domain) for this lane's query
  float l_run = 0.f;        // this lane's partial sum of P~ in fp32 (its half of the keys): LSE
  float lb_run = 0.f;       // the same sum over P~ as rounded to bf16 for the MFMA: O's divisor

  auto compute_tile = [&](int j, const unsigned char* stage) {
    const int key0 = j * BC;
    // a5: a wave whose rows all precede this tile's first key, or whose rows are all past
    // the end of the sequence, has nothing to add here.
    if ((CAUSAL && key0 > qw0 + 31 + diag) || qw0 >= seq_len) return;
    const unsigned char* ks = stage;

    // ---- a4: S^T = K_j Q^T ----------------------------------------------------------
    f32x16 s[TL::NKB];
#pragma unroll
    for (int kb = 0; kb < TL::NKB; ++kb) s[kb] = (f32x16){};
    if constexpr (RING) {
      // Nested in the loop over blocks the scheduling-group hints do not hold, so the K
      // fragments are read LA ahead from a register ring (fences keep the order).
      constexpr int NF = TL::NKB * TL::NKC;
      constexpr int SR = LA > 0 ? (LA < NF ? LA : NF) : 1;
      bf16x8 kr[SR];
      auto rd = [&](int f) {
        const int kb = f / TL::NKC, kc = f % TL::NKC;
        kr[f % SR] = *(const bf16x8*)(ks + kb * 32 * TL::ROWB + (kc >> 3) * 256 + kaddr[kc & 7]);
      };
#pragma unroll
      for (int f = 0; f < SR; ++f) rd(f);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int kb = f / TL::NKC, kc = f % TL::NKC;
        __builtin_amdgcn_sched_barrier(0);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[f % SR], qf[kc], s[kb], 0, 0, 0);
        if (f + SR < NF) rd(f + SR);
      }
      __builtin_amdgcn_sched_barrier(0);
    } else if constexpr (TL::NKB == 1 && LA > 0) {
      // One 32-key chain: scheduling-group hints do not move its K reads ahead, so they are
      // issued explicitly, SR fragments ahead of their MFMAs, from a ring held in registers
      // (the fences keep the order).
      constexpr int SR = LA < TL::NKC ? LA : TL::NKC;
      bf16x8 kr[SR];
      auto rd = [&](int kc) {
        kr[kc % SR] = *(const bf16x8*)(ks + (kc >> 3) * 256 + kaddr[kc & 7]);
      };
#pragma unroll
      for (int kc = 0; kc < SR; ++kc) rd(kc);
#pragma unroll
      for (int kc = 0; kc < TL::NKC; ++kc) {
        __builtin_amdgcn_sched_barrier(0);
        s[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[kc % SR], qf[kc], s[0], 0, 0, 0);
        if (kc + SR < TL::NKC) rd(kc + SR);
      }
      __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll
      for (int kb = 0; kb < TL::NKB; ++kb) {
#pragma unroll
        for (int kc = 0; kc < TL::NKC; ++kc) {
          const bf16x8 a = *(const bf16x8*)(ks + kb * 32 * TL::ROWB + (kc >> 3) * 256 + kaddr[kc & 7]);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kc], s[kb], 0, 0, 0);
        }
      }
      if constexpr (LA > 0) {
        // LDS latency: keep LA fragment reads in flight ahead of the MFMA chains.
        constexpr int NF = TL::NKB * TL::NKC;
        __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (f + LA < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
    }

    // ---- a5: mask on diagonal and ragged tiles only -----------------------------------
    // Entry (kb, r) of this lane is key key0 + koffs with koffs = kb*32 + 8*(r/4) + 4*hl + r%4.
    // It is dead when koffs - 4*hl exceeds thr (causal: key > query; ragged: key >= length),
    // a per-lane threshold; the sign of thr - const selects -inf with one bitfield insert.
    if ((CAUSAL && key0 + BC - 1 > qw0 + diag) || key0 + BC > seq_k) {
      // The lane-derived terms are taken afresh here: kept from the thread id they would
      // stay live across the tile loop, only for the diagonal and ragged tiles.
      const int ln = wave_lane();
      const int hm = ln >> 5;
      int thr = seq_k - 1 - key0 - 4 * hm;
      if (CAUSAL) thr = min(thr, qw0 + (ln & 31) + diag - key0 - 4 * hm);
#pragma unroll
      for (int kb = 0; kb < TL::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kc = kb * 32 + 8 * (r >> 2) + (r & 3);
          const uint32_t dead = (uint32_t)((thr - kc) >> 31);          // all ones if kc > thr
          const uint32_t bits = __float_as_uint(s[kb][r]);
          s[kb][r] = __uint_as_float((bits & ~dead) | (0xff800000u & dead));   // -inf
        }
    }

    // ---- a6: online softmax (fp32) --------------------------------------------------
    // pw[c] holds P~ for PV contraction step c as 4 packed bf16 pairs. Two row sums are
    // kept: the fp32 sum of P~ (for the LSE) and the sum of P~ as rounded to bf16, i.e.
    // of exactly the weights the PV product consumes, so that O = O~ / l is a normalised
    // average of V rows even where one key dominates a row.
    u32x4 pw[TL::NPC];
    float rsb;   // the bf16-rounded sum of the last form_p
    auto form_p = [&](float m_ref) {
      float rsum = 0.f;
      rsb = 0.f;
#pragma unroll
      for (int c = 0; c < TL::NPC; ++c) {
        const int kb = c >> 1, r0 = (c & 1) * 8;
        float e[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          e[u] = __builtin_amdgcn_exp2f(fmaf(s[kb][r0 + u], p.c, -m_ref));
          rsum += e[u];
        }
        pw[c] = (u32x4){pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]),
                        pack_bf16x2(e[4], e[5]), pack_bf16x2(e[6], e[7])};
#pragma unroll
        for (int w = 0; w < 4; ++w) rsb = sum_bf16x2(pw[c][w], rsb);
      }
      return rsum;
    };
    auto tile_max = [&]() {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < TL::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      return halves_max(mx) * p.c;   // -inf stays -inf (c > 0)
    };
    // Move the reference max to m_new (per lane), rescaling l and O~ by 2^(m_run - m_new).
    auto rescale_to = [&](float m_new) {
      const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);   // 0 when m_run = -inf
      l_run *= alpha;
      lb_run *= alpha;
#pragma unroll
      for (int db = 0; db < TL::NDB; ++db) oacc[db] *= alpha;
      m_run = m_new;
    };
    float rs;
    if (MODE == kOptimistic) {
      rs = form_p(m_run == -INFINITY ? 0.f : m_run);
      // Slow path: the row's first tile, or a tile whose P~ grew too large (rs may be inf).
      if (__builtin_amdgcn_ballot_w64(!(rs <= kOptLimit) || m_run == -INFINITY)) {
        rescale_to(fmaxf(m_run, tile_max()));
        rs = form_p(m_run == -INFINITY ? 0.f : m_run);
      }
    } else if (MODE == kLazy) {
      const float mt = tile_max();
      const bool need = mt > m_run + kLazyTau;    // false when the tile is fully masked
      if (__builtin_amdgcn_ballot_w64(need)) rescale_to(need ? mt : m_run);
      rs = form_p(m_run == -INFINITY ? 0.f : m_run);
    } else {
      const float m_new = fmaxf(m_run, tile_max());
      const float m_ref = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_ref);
      const bool grew = m_new > m_run;
      l_run *= alpha;
      lb_run *= alpha;
      // Skip the O~ rescale when no row of the wave changed its max (alpha == 1 exactly).
      if (__builtin_amdgcn_ballot_w64(grew)) {
#pragma unroll
        for (int db = 0; db < TL::NDB; ++db) oacc[db] *= alpha;
      }
      m_run = m_new;
      rs = form_p(m_ref);
    }
    l_run += rs;
    lb_run += rsb;

    // ---- a7: O~^T += V_j^T P~^T -----------------------------------------------------
    if constexpr (RING) {
      // V^T fragments read LA ahead from a register ring.
      constexpr int NF = TL::NPC * TL::NDB;
      constexpr int VR = LA > 0 ? (LA < NF ? LA : NF) : 1;
      bf16x8 vq[VR];
      auto rdv = [&](int f) {
        const int c = f / TL::NDB, db = f % TL::NDB;
        const unsigned char* va = stage + vaddr[db & 3] + (db >> 2) * 256 + 16 * c * TL::ROWB;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, va));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, va + 8 * TL::ROWB));
        vq[f % VR] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
#pragma unroll
      for (int f = 0; f < VR; ++f) rdv(f);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int c = f / TL::NDB, db = f % TL::NDB;
        __builtin_amdgcn_sched_barrier(0);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vq[f % VR], as_bf16x8(pw[c]), oacc[db], 0, 0, 0);
        if (f + VR < NF) rdv(f + VR);
      }
      __builtin_amdgcn_sched_barrier(0);
    } else {
#pragma unroll
      for (int c = 0; c < TL::NPC; ++c) {
        const bf16x8 pf = as_bf16x8(pw[c]);
#pragma unroll
        for (int db = 0; db < TL::NDB; ++db) {
          const unsigned char* va = stage + vaddr[db & 3] + (db >> 2) * 256 + 16 * c * TL::ROWB;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, va));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, va + 8 * TL::ROWB));
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf, oacc[db], 0, 0, 0);
        }
      }
      if constexpr (LA > 0) {
        constexpr int NF = TL::NPC * TL::NDB;       // V^T fragments per tile
        constexpr int RPF = 2;                      // transposed LDS reads per fragment
        __builtin_amdgcn_sched_group_barrier(0x100, LA * RPF, 0);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (f + LA < NF) __builtin_amdgcn_sched_group_barrier(0x100, RPF, 0);
        }
      }
    }
  };

  // ---- the key/value loop: one barrier per tile ----------------------------------------
  // Iteration j begins after a barrier that publishes tile j in its stage and certifies
  // every wave has finished tile j-1, whose stage now takes tile j+1: its direct loads
  // start, tile j is computed, the loads are waited for, and the next barrier follows.
  auto iteration = [&](int j, unsigned char* cur, unsigned char* nxt) {
    if (j + 1 < nt) dma_tile(j + 1, nxt);
    compute_tile(j, cur);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  if (nt > 0) dma_tile(0, lds0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int j = 0; j < nt; j += 2) {
    iteration(j, lds0, lds1);
    if (j + 1 < nt) iteration(j + 1, lds1, lds0);
  }

  // ---- a8: epilogue: O = O~ / l, LSE = (m + log2 l) ln 2 --------------------------------
  // O divides by the sum of the bf16 weights the PV product used; the LSE takes the fp32 sum.
  const float l_tot = halves_sum(l_run);
  const float lb_tot = halves_sum(lb_run);
  if (qrow < seq_len) {
    const float inv = lb_tot > 0.f ? 1.f / lb_tot : 0.f;
    uint16_t* orow = p.o + (orow0 + (size_t)qrow) * dg;
#pragma unroll
    for (int db = 0; db < TL::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w = {pack_bf16x2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv),
                   pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
        if (db * 32 + 8 * g + 4 * hl < dg) *(u32x2*)(orow + db * 32 + 8 * g + 4 * hl) = w;
      }
    if (hl == 0) {
      p.lse[orow0 + (size_t)qrow] =
          l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

// One workgroup per row block. OCC: waves per SIMD the kernel is built for (its registers
// are limited to 512 / OCC per lane); more resident waves let one wave's softmax run while
// another's MFMAs occupy the matrix core.
template <int D, int BC, bool CAUSAL, bool VARLEN, int MODE, int LA, int NW = 4,
          int OCC = (D == 256 ? 1 : 2)>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(OCC, OCC)))
void fa2_fwd_kernel(Params p) {
  fwd_block<D, BC, CAUSAL, VARLEN, MODE, LA, NW, false>(p, (int)blockIdx.x);
}

// ---- persistent variant ----------------------------------------------------------------
// The same row-block computation (fwd_block, with its fragment reads in register rings), run
// by as many workgroups as the CUs hold. Each workgroup takes row blocks from a work queue in
// global memory (run_work_queue) until none is left, so one block's start follows the
// previous one's end on the CU without a new workgroup's dispatch and start-up. With the
// XCD-aware order there is one queue per XCD (workgroup w serves queue w % 8, the XCD the
// round-robin dispatch places it on, and takes the ids x, x + 8, ... of its XCD's heads);
// otherwise one queue.
template <int D, int BC, bool CAUSAL, bool VARLEN, int MODE, int LA, int NW = 4,
          int OCC = (D == 256 ? 1 : 2)>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(OCC, OCC)))
void fa2_fwd_kernel_persist(Params p, unsigned int* ctr, int total) {
  run_work_queue(ctr, p.heads_per_xcd > 0 ? 8 : 1, total,
                 [&](int id) { fwd_block<D, BC, CAUSAL, VARLEN, MODE, LA, NW, true>(p, id); });
}

// ---- ping-pong variant ---------------------------------------------------------------
// Same method and per-wave tiles (32 query rows per wave, S^T / O^T formulation), with eight
// waves per workgroup (256 query rows) arranged so that the two waves sharing a SIMD work in
// opposite phases: while one runs matrix-core work (the PV product of tile j-1 and the S
// product of tile j), the other runs the softmax VALU work of a tile, and all eight waves
// meet at a barrier between phases. Every wave runs the same sequence
//     [MFMA phase: PV(j-1), S(j)]  barrier  [VALU phase: softmax(j)]  barrier
// and group B (waves 4..7) executes one extra barrier before it, group A (waves 0..3) one
// after it, so B trails A by exactly one phase and their MFMA and VALU phases alternate.
// K/V tiles are staged by direct loads into a ring of four LDS stages. A wave issues its
// share of tile j+2 at the start of its MFMA phase j and waits for tile j+1 at the end of
// it. In global phases, tile t is issued in phase 2t-4 (group A) or 2t-3 (group B), is
// complete by the end of phase 2t-1, and is last read in phase 2t+3 (group B's PV(t)), so
// the stage of tile t-4, last read in phase 2t-5, is free.
template <int D, int BC>
struct TilePP {
  static constexpr int WAVES = 8;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BR = 32 * WAVES;
  static constexpr int ROWB = 2 * D;
  static constexpr int TILEB = BC * ROWB;
  static constexpr int STAGEB = 2 * TILEB;                  // K tile then V tile
  static constexpr int NSTAGE = 4;
  static constexpr int LDS_BYTES = NSTAGE * STAGEB;
  static constexpr int DMA_PER_WAVE = TILEB / 1024 / WAVES;
  static constexpr int NKB = BC / 32;
  static constexpr int NKC = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int NPC = BC / 16;
  static_assert(D == 64 || D == 128, "head dim");
  static_assert(BC % 32 == 0 && TILEB % (1024 * WAVES) == 0 && DMA_PER_WAVE >= 1, "tile shape");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget");
  __device__ static int kswz(int row) { return Tile<D, BC>::kswz(row); }
  __device__ static int vswz(int row) { return Tile<D, BC>::vswz(row); }
};

template <int D, int BC, bool CAUSAL, bool VARLEN, int LA>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void fa2_fwd_kernel_pp(Params p) {
  using TL = TilePP<D, BC>;
  __shared__ __attribute__((aligned(1024))) unsigned char lds[TL::LDS_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int grp = wave >> 2;    // 0: group A, 1: group B (one phase behind)
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  // ---- a1: work decode ----------------------------------------------------------------
  int bh, i;
  decode_block<CAUSAL>(p, (int)blockIdx.x, bh, i);
  const int bi = bh / p.H;
  const int h = bh - bi * p.H;
  int seq_len, seq_k;
  const int hk = h / p.g;
  size_t row0, kvrow0;
  if (VARLEN) {
    int a = p.cu_seqlens[bi];
    int e = p.cu_seqlens[bi + 1];
    a = min(max(a, 0), p.T);
    e = min(max(e, a), p.T);
    seq_len = e - a;
    seq_k = seq_len;
    row0 = (size_t)h * (size_t)p.T + (size_t)a;
    kvrow0 = (size_t)hk * (size_t)p.T + (size_t)a;
  } else {
    seq_len = p.N;
    seq_k = p.Nk;
    row0 = (size_t)bh * (size_t)p.N;
    kvrow0 = ((size_t)bi * (size_t)p.Hkv + (size_t)hk) * (size_t)p.Nk;
  }
  // Split-KV: split s of the launch owns keys [s*split_len, (s+1)*split_len) and writes its
  // partial O and LSE to part s of the output (rows offset by s*part_rows).
  const int ks0 = VARLEN ? 0 : (int)blockIdx.y * p.split_len;
  if (!VARLEN) {
    seq_k = max(min(p.split_len, seq_k - ks0), 0);
    kvrow0 += (size_t)ks0;
  }
  const int diag = p.diag - ks0;
  const size_t orow0 = row0 + (VARLEN ? 0 : (size_t)blockIdx.y * (size_t)p.part_rows);
  const int q0 = i * TL::BR;
  if (q0 >= seq_len) return;

  const int dg = p.dg;            // row pitch of Q, K, V, O in elements
  const int growb = 2 * dg;       // ... in bytes
  const uint16_t* __restrict__ qh = p.q + row0 * dg;
  const unsigned char* kh = (const unsigned char*)(p.k + kvrow0 * dg);
  const unsigned char* vh = (const unsigned char*)(p.v + kvrow0 * dg);
  const int kv_end = max(CAUSAL ? min(seq_k, q0 + TL::BR + diag) : seq_k, 0);
  const int nt = (kv_end + BC - 1) / BC;

  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;
  // Tiles this wave computes: causal tile j matters iff its first key <= the wave's last row.
  const int last_key = qw0 + 31 + diag;
  const int ntw = (qw0 >= seq_len) ? 0
                  : (CAUSAL ? (last_key < 0 ? 0 : min(nt, last_key / BC + 1)) : nt);

  // ---- a2: Q^T fragments ----------------------------------------------------------------
  bf16x8 qf[TL::NKC];
  load_q_fragments<TL::NKC>(qf, qh, qrow, seq_len, dg, hl, p.qflip);

  // ---- a3: direct global -> LDS staging into the stage ring -----------------------------
  int drow[TL::DMA_PER_WAVE];
  uint32_t koff[TL::DMA_PER_WAVE];
  uint32_t voff[TL::DMA_PER_WAVE];
#pragma unroll
  for (int d = 0; d < TL::DMA_PER_WAVE; ++d) {
    const int b = wave * TL::DMA_PER_WAVE + d;
    const int o = b * 1024 + lane * 16;
    const int r = o / TL::ROWB;
    const int pch = (o % TL::ROWB) / 16;
    drow[d] = r;
    // Padded columns (logical chunk beyond dg) load a real chunk of the same row: finite, and
    // multiplied by Q's zero columns (K) or landing in unwritten O columns (V).
    koff[d] = r * growb + (((pch ^ TL::kswz(r)) % (dg / 8)) * 16);
    voff[d] = r * growb + (((pch ^ TL::vswz(r)) % (dg / 8)) * 16);
  }
  const uint32_t lds_base = lds_addr(lds);
  auto dma_tile = [&](int j) {
    const int key0 = j * BC;
    const unsigned char* kt = kh + (size_t)key0 * growb;
    const unsigned char* vt = vh + (size_t)key0 * growb;
    const uint32_t st = lds_base + (uint32_t)(j & (TL::NSTAGE - 1)) * TL::STAGEB;
    const uint32_t ks_a = st + wave * TL::DMA_PER_WAVE * 1024;
    const uint32_t vs_a = st + TL::TILEB + wave * TL::DMA_PER_WAVE * 1024;
    if (key0 + BC <= seq_k) {
#pragma unroll
      for (int d = 0; d < TL::DMA_PER_WAVE; ++d) {
        dma16(kt, koff[d], ks_a + d * 1024);
        dma16(vt, voff[d], vs_a + d * 1024);
      }
    } else {
      const int last = seq_k - 1 - key0;   // rows past the end re-read the last valid row
#pragma unroll
      for (int d = 0; d < TL::DMA_PER_WAVE; ++d) {
        const uint32_t back = (uint32_t)(drow[d] - min(drow[d], last)) * growb;
        dma16(kt, koff[d] - back, ks_a + d * 1024);
        dma16(vt, voff[d] - back, vs_a + d * 1024);
      }
    }
  };

  int kaddr[TL::NKC];
#pragma unroll
  for (int kc = 0; kc < TL::NKC; ++kc)
    kaddr[kc] = l32 * TL::ROWB + (((2 * kc + hl) ^ TL::kswz(l32)) * 16);
  const int vr = 4 * hl + ((lane & 15) >> 2);
  int vaddr[TL::NDB];
#pragma unroll
  for (int db = 0; db < TL::NDB; ++db) {
    const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    vaddr[db] = TL::TILEB + vr * TL::ROWB + (((col >> 3) ^ TL::vswz(vr)) * 16) + (col & 7) * 2;
  }

  // ---- running state ------------------------------------------------------------------
  f32x16 oacc[TL::NDB];
#pragma unroll
  for (int db = 0; db < TL::NDB; ++db) oacc[db] = (f32x16){};
  float m_run = -INFINITY;
  float l_run = 0.f;      // fp32 sum of P~ (LSE)
  float lb_run = 0.f;     // sum of P~ as rounded to bf16 (O's divisor)
  f32x16 s[TL::NKB];      // S of the tile the next VALU phase works on
  u32x4 pw[TL::NPC];      // P~ (bf16 pairs) of the tile the next MFMA phase multiplies

  auto stage_ptr = [&](int j) { return lds + (j & (TL::NSTAGE - 1)) * TL::STAGEB; };

  // MFMA phase: PV of tile jp (if any) and S of tile js (if any), interleaved.
  auto mfma_phase = [&](int jp, int js) {
    const bool do_pv = jp >= 0 && jp < ntw;
    const bool do_s = js < ntw;
    if (do_pv) {
      const unsigned char* st = stage_ptr(jp);
#pragma unroll
      for (int c = 0; c < TL::NPC; ++c) {
        const bf16x8 pf = as_bf16x8(pw[c]);
#pragma unroll
        for (int db = 0; db < TL::NDB; ++db) {
          const unsigned char* va = st + vaddr[db] + 16 * c * TL::ROWB;
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, va));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, va + 8 * TL::ROWB));
          const bf16x8 a = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pf, oacc[db], 0, 0, 0);
        }
      }
      if constexpr (LA > 0) {
        constexpr int NF = TL::NPC * TL::NDB;
        __builtin_amdgcn_sched_group_barrier(0x100, 2 * LA, 0);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (f + LA < NF) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
      }
    }
    if (do_s) {
      const unsigned char* ks = stage_ptr(js);
#pragma unroll
      for (int kb = 0; kb < TL::NKB; ++kb) {
        s[kb] = (f32x16){};
#pragma unroll
        for (int kc = 0; kc < TL::NKC; ++kc) {
          const bf16x8 a = *(const bf16x8*)(ks + kb * 32 * TL::ROWB + kaddr[kc]);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[kc], s[kb], 0, 0, 0);
        }
      }
      if constexpr (LA > 0) {
        constexpr int NF = TL::NKB * TL::NKC;
        __builtin_amdgcn_sched_group_barrier(0x100, LA, 0);
#pragma unroll
        for (int f = 0; f < NF; ++f) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (f + LA < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
      }
    }
  };

  // VALU phase: mask and online softmax of tile j (lazy reference max: the tile's row max
  // is taken, and m, l and O~ move only when it exceeds m by 2^kLazyTau). P~ is formed in
  // place in fp32, then packed to bf16 for the next MFMA phase.
  auto valu_phase = [&](int j) {
    if (j >= ntw) return;
    const int key0 = j * BC;
    if ((CAUSAL && key0 + BC - 1 > qw0 + diag) || key0 + BC > seq_k) {
      int thr = seq_k - 1 - key0 - 4 * hl;
      if (CAUSAL) thr = min(thr, qrow + diag - key0 - 4 * hl);
#pragma unroll
      for (int kb = 0; kb < TL::NKB; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kc = kb * 32 + 8 * (r >> 2) + (r & 3);
          const uint32_t dead = (uint32_t)((thr - kc) >> 31);
          const uint32_t bits = __float_as_uint(s[kb][r]);
          s[kb][r] = __uint_as_float((bits & ~dead) | (0xff800000u & dead));
        }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < TL::NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    const float mt = halves_max(mx) * p.c;
    const bool need = mt > m_run + kLazyTau;   // false for a fully masked tile
    if (__builtin_amdgcn_ballot_w64(need)) {
      const float m_new = need ? mt : m_run;
      const float alpha = need ? __builtin_amdgcn_exp2f(m_run - m_new) : 1.f;   // 0 if m_run = -inf
      l_run *= alpha;
      lb_run *= alpha;
#pragma unroll
      for (int db = 0; db < TL::NDB; ++db) oacc[db] *= alpha;
      m_run = m_new;
    }
    const float m_ref = (m_run == -INFINITY) ? 0.f : m_run;
    float rsum = 0.f, rsb = 0.f;
#pragma unroll
    for (int c = 0; c < TL::NPC; ++c) {
      const int kb = c >> 1, r0 = (c & 1) * 8;
      float e[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        e[u] = __builtin_amdgcn_exp2f(fmaf(s[kb][r0 + u], p.c, -m_ref));
        rsum += e[u];
      }
      pw[c] = (u32x4){pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]),
                      pack_bf16x2(e[4], e[5]), pack_bf16x2(e[6], e[7])};
#pragma unroll
      for (int w = 0; w < 4; ++w) rsb = sum_bf16x2(pw[c][w], rsb);
    }
    l_run += rsum;
    lb_run += rsb;
  };

  // ---- the phase loop ------------------------------------------------------------------
  if (nt > 0) dma_tile(0);
  if (nt > 1) dma_tile(1);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (grp == 1) __syncthreads();        // group B trails group A by one phase
  for (int j = 0; j <= nt; ++j) {
    const bool more = j + 2 < nt;
    if (more) dma_tile(j + 2);
    mfma_phase(j - 1, j);
    // Tile j+1 must be in LDS before the barrier; tile j+2's loads may stay in flight.
    if (more) {
      if constexpr (2 * TL::DMA_PER_WAVE == 4) asm volatile("s_waitcnt vmcnt(4)" ::: "memory");
      else if constexpr (2 * TL::DMA_PER_WAVE == 2) asm volatile("s_waitcnt vmcnt(2)" ::: "memory");
      else asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();
    valu_phase(j);
    __syncthreads();
  }
  if (grp == 0) __syncthreads();

  // ---- a8: epilogue ------------------------------------------------------------------
  const float l_tot = halves_sum(l_run);
  const float lb_tot = halves_sum(lb_run);
  if (qrow < seq_len) {
    const float inv = lb_tot > 0.f ? 1.f / lb_tot : 0.f;
    uint16_t* orow = p.o + (orow0 + (size_t)qrow) * dg;
#pragma unroll
    for (int db = 0; db < TL::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w = {pack_bf16x2(oacc[db][4 * g + 0] * inv, oacc[db][4 * g + 1] * inv),
                   pack_bf16x2(oacc[db][4 * g + 2] * inv, oacc[db][4 * g + 3] * inv)};
        if (db * 32 + 8 * g + 4 * hl < dg) *(u32x2*)(orow + db * 32 + 8 * g + 4 * hl) = w;
      }
    if (hl == 0) {
      p.lse[orow0 + (size_t)qrow] =
          l_tot > 0.f ? (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
    }
  }
}

// ---- host side ------------------------------------------------------------------------

typedef const void* KernelFn;

struct Variant {
  const char* name;
  int d;
  int br;
  int bc;
  int lds;
  int threads;
  KernelFn fixed[2];   // [causal]
  KernelFn varlen[2];  // [causal]
  int wg_per_cu = 0;   // > 0: persistent form, launched with this many workgroups per CU
  // Persistent form: the one-block-per-workgroup kernels that run the same tiles, for
  // split-KV launches and launches captured into a graph.
  KernelFn plain_fixed[2] = {nullptr, nullptr};
  KernelFn plain_varlen[2] = {nullptr, nullptr};
};

template <int D, int BC, int MODE, int LA = 0, int NW = 4, int OCC = (D == 256 ? 1 : 2)>
Variant make_variant(const char* name) {
  using TL = Tile<D, BC, NW>;
  Variant v;
  v.threads = TL::THREADS;
  v.name = name;
  v.d = D;
  v.br = TL::BR;
  v.bc = BC;
  v.lds = TL::LDS_BYTES;
  v.fixed[0] = (KernelFn)&fa2_fwd_kernel<D, BC, false, false, MODE, LA, NW, OCC>;
  v.fixed[1] = (KernelFn)&fa2_fwd_kernel<D, BC, true, false, MODE, LA, NW, OCC>;
  v.varlen[0] = (KernelFn)&fa2_fwd_kernel<D, BC, false, true, MODE, LA, NW, OCC>;
  v.varlen[1] = (KernelFn)&fa2_fwd_kernel<D, BC, true, true, MODE, LA, NW, OCC>;
  return v;
}

template <int D, int BC, int MODE, int LA, int NW, int OCC>
Variant make_variant_persist(const char* name) {
  Variant v = make_variant<D, BC, MODE, LA, NW, OCC>(name);
  v.plain_fixed[0] = v.fixed[0];
  v.plain_fixed[1] = v.fixed[1];
  v.plain_varlen[0] = v.varlen[0];
  v.plain_varlen[1] = v.varlen[1];
  v.fixed[0] = (KernelFn)&fa2_fwd_kernel_persist<D, BC, false, false, MODE, LA, NW, OCC>;
  v.fixed[1] = (KernelFn)&fa2_fwd_kernel_persist<D, BC, true, false, MODE, LA, NW, OCC>;
  v.varlen[0] = (KernelFn)&fa2_fwd_kernel_persist<D, BC, false, true, MODE, LA, NW, OCC>;
  v.varlen[1] = (KernelFn)&fa2_fwd_kernel_persist<D, BC, true, true, MODE, LA, NW, OCC>;
  v.wg_per_cu = 4 * OCC / NW;
  return v;
}

template <int D, int BC, int LA>
Variant make_variant_pp(const char* name) {
  using TL = TilePP<D, BC>;
  Variant v;
  v.threads = TL::THREADS;
  v.name = name;
  v.d = D;
  v.br = TL::BR;
  v.bc = BC;
  v.lds = TL::LDS_BYTES;
  v.fixed[0] = (KernelFn)&fa2_fwd_kernel_pp<D, BC, false, false, LA>;
  v.fixed[1] = (KernelFn)&fa2_fwd_kernel_pp<D, BC, true, false, LA>;
  v.varlen[0] = (KernelFn)&fa2_fwd_kernel_pp<D, BC, false, true, LA>;
  v.varlen[1] = (KernelFn)&fa2_fwd_kernel_pp<D, BC, true, true, LA>;
  return v;
}

// Variant 0 of each head dimension is the default; the others exist for tuning and tests.
const Variant* variants_for(int d, int* count) {
  // d = 64: the O~ accumulator is half that of d = 128, so a 64-key tile fits in 128
  // registers and four waves share each SIMD (two 8-wave workgroups per CU, 32 KB of LDS
  // each); the softmax work, which per flop is twice that of d = 128, then overlaps the
  // matrix work of the other waves.
  static const Variant v64[] = {
      make_variant<64, 64, kOptimistic, 4, 8, 4>("d64_w8_bc64_occ4_la4"),
      make_variant<64, 128, kOptimistic, 4>("d64_bc128_opt_la4"),
      make_variant<64, 128, kOptimistic>("d64_bc128_opt"),
      make_variant<64, 128, kLazy, 4>("d64_bc128_lazy_la4"),
      make_variant<64, 128, kExact>("d64_bc128_exact"),
      make_variant_pp<64, 64, 4>("d64_pp_bc64_la4"),
      make_variant<64, 128, kOptimistic, 4, 8>("d64_w8_bc128_opt_la4"),
      make_variant<64, 64, kOptimistic, 4, 4, 3>("d64_bc64_occ3_la4")};
  static const Variant v128[] = {
      make_variant<128, 64, kOptimistic, 4, 8>("d128_w8_bc64_opt_la4"),
      make_variant<128, 64, kOptimistic, 4>("d128_bc64_opt_la4"),
      make_variant<128, 64, kOptimistic>("d128_bc64_opt"),
      make_variant<128, 64, kLazy, 4>("d128_bc64_lazy_la4"),
      make_variant<128, 64, kExact>("d128_bc64_exact"),
      make_variant_pp<128, 64, 4>("d128_pp_bc64_la4"),
      make_variant<128, 32, kOptimistic, 4, 4, 3>("d128_bc32_occ3_la4"),
      make_variant_persist<128, 64, kOptimistic, 4, 8, 2>("d128_w8_bc64_persist")};
  // d = 256: the O~ accumulator alone is 128 registers. With 32-key tiles (and the K/V read
  // offsets past the 16th chunk of a row folded into immediates) a wave fits in 256
  // registers, so two waves share each SIMD in an 8-wave workgroup; the 64-key forms run one
  // wave per SIMD. The ping-pong family, which needs two waves per SIMD at 64-key tiles, has
  // no d = 256 member.
  static const Variant v256[] = {
      make_variant<256, 32, kOptimistic, 4, 8, 2>("d256_w8_bc32_occ2_la4"),
      make_variant<256, 64, kOptimistic, 4>("d256_bc64_opt_la4"),
      make_variant<256, 32, kOptimistic, 4>("d256_bc32_opt_la4"),
      make_variant<256, 64, kExact>("d256_bc64_exact"),
      make_variant<256, 32, kOptimistic, 4, 4, 2>("d256_bc32_occ2_la4")};
  if (d == 64) {
    *count = (int)(sizeof(v64) / sizeof(v64[0]));
    return v64;
  }
  if (d == 256) {
    *count = (int)(sizeof(v256) / sizeof(v256[0]));
    return v256;
  }
  if (d == 128) {
    *count = (int)(sizeof(v128) / sizeof(v128[0]));
    return v128;
  }
  *count = 0;
  return nullptr;
}

bool aligned(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

// Head dimensions the forward accepts: any multiple of 8 up to 256. The kernels exist for
// D = 64, 128 and 256; a smaller d runs on the next one with its columns padded (zero in Q,
// unwritten in O), so its matrix work is that of the padded width.
bool fwd_head_dim(int d) { return d >= 8 && d <= 256 && d % 8 == 0; }
int padded_dim(int d) { return d <= 64 ? 64 : d <= 128 ? 128 : 256; }

// The variant fa2_fwd_varlen runs: at (padded) d = 128 the persistent form, whose work queue
// skips the row blocks past the end of shorter sequences instead of launching a workgroup
// for each; variant 0 otherwise.
int default_varlen_variant(int d) {
  if (!fwd_head_dim(d) || padded_dim(d) != 128) return 0;
  int count = 0;
  const Variant* vs = variants_for(128, &count);
  for (int i = 0; i < count; ++i)
    if (vs[i].wg_per_cu > 0) return i;
  return 0;
}

int check_common(const void* q, const void* k, const void* v, const void* o, const float* lse,
                 int d, float scale, int variant, const Variant** out) {
  if (!q || !k || !v || !o || !lse) return FA2_ERR_NULL_PTR;
  if (!fwd_head_dim(d)) return FA2_ERR_UNSUPPORTED_HEADDIM;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(o, 16) || !aligned(lse, 4))
    return FA2_ERR_MISALIGNED;
  if (!isfinite(scale)) return FA2_ERR_BAD_SCALE;
  int count = 0;
  const Variant* vs = variants_for(padded_dim(d), &count);
  if (variant < 0 || variant >= count) return FA2_ERR_BAD_VARIANT;
  *out = &vs[variant];
  return FA2_OK;
}

}  // namespace

// Work-queue counters of the persistent form: kQueueSlots sets of 16 words (8 queues and the
// count of finished workgroups), zero when the library is loaded. Every launch takes the next
// set in turn, and its last workgroup returns the set to zero. Launches in flight at the
// same time (other streams, graphs) use different sets as long as fewer than kQueueSlots
// persistent launches run at once on a device.
constexpr int kQueueSlots = 1024;
static __device__ unsigned int persist_ctr[kQueueSlots * 16];

namespace {

constexpr int kMaxQueueDevices = 64;
std::mutex persist_mu;
unsigned int* persist_base[kMaxQueueDevices];   // device address of persist_ctr, per device
unsigned long long persist_next[kMaxQueueDevices];

}  // namespace

int fa2_internal::queue_counters(int dev, unsigned int** out) {
  if (dev < 0 || dev >= kMaxQueueDevices) return FA2_ERR_NO_DEVICE;
  std::lock_guard<std::mutex> lock(persist_mu);
  if (!persist_base[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(persist_ctr)) != hipSuccess || !ptr) return FA2_ERR_NO_DEVICE;
    persist_base[dev] = (unsigned int*)ptr;
  }
  *out = persist_base[dev] + 16 * (persist_next[dev]++ % kQueueSlots);
  return FA2_OK;
}

namespace {

int launch(const Variant& var, bool varlen, bool causal, Params& p, int num_wg, void* stream,
           int grid_y = 1) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FA2_ERR_NO_DEVICE;
  KernelFn fn = varlen ? var.varlen[causal ? 1 : 0] : var.fixed[causal ? 1 : 0];
  // A graph would keep the counter set it captured and replay it while later launches take
  // the same set in turn, so a launch under stream capture takes the one-block-per-workgroup
  // kernel instead (same tiles, same results).
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (var.wg_per_cu > 0 && hipStreamIsCapturing((hipStream_t)stream, &cap) != hipSuccess)
    return FA2_ERR_LAUNCH;
  if (var.wg_per_cu > 0 && grid_y == 1 && cap == hipStreamCaptureStatusNone) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return FA2_ERR_NO_DEVICE;
    unsigned int* ctr = nullptr;
    const int st = fa2_internal::queue_counters(dev, &ctr);
    if (st != FA2_OK) return st;
    int total = num_wg;
    const int grid = std::min(num_wg, cus * var.wg_per_cu);
    void* pargs[] = {&p, &ctr, &total};
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)grid), dim3((unsigned)var.threads), pargs, 0,
                                   (hipStream_t)stream);
    return e == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
  }
  if (var.wg_per_cu > 0) fn = varlen ? var.plain_varlen[causal ? 1 : 0] : var.plain_fixed[causal ? 1 : 0];
  void* args[] = {&p};
  hipError_t e = hipLaunchKernel(fn, dim3((unsigned)num_wg, (unsigned)grid_y), dim3((unsigned)var.threads), args, 0,
                                 (hipStream_t)stream);
  return e == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}

void fill_scale(Params& p, float scale) {
  // A zero scale gives uniform attention; a tiny positive c reproduces that (every score
  // times c rounds to 0) while keeping -inf * c = -inf for masked entries.
  p.c = fmaxf(fabsf(scale) * kLog2e, 1e-30f);
  p.qflip = scale < 0.f ? 0x80008000u : 0u;
}

int heads_per_xcd(long long nbh) { return (nbh % 8 == 0) ? (int)(nbh / 8) : 0; }

// Keys per split-KV piece (a multiple of the variant's key tile) and the number of pieces.
void split_pieces(int N_k, int num_splits, int bc, int* split_len, int* ns) {
  *split_len = N_k;
  *ns = 1;
  if (num_splits > 1 && N_k > 0) {
    const int per = (N_k + num_splits - 1) / num_splits;
    *split_len = (per + bc - 1) / bc * bc;
    *ns = (N_k + *split_len - 1) / *split_len;
  }
}

// Shared body of fa2_fwd_chunk (num_splits == 1) and fa2_fwd_splitkv. With splits, the keys are
// cut into ns contiguous pieces of split_len keys (a multiple of the key tile), one launch
// computes every (row block, piece) pair into the caller's o_parts / lse_parts, and the LSE
// merge combines the pieces into o / lse.
// With dry_run the call stops after validation, before any HIP call.
int fwd_chunk_impl(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                   int H_kv, int N_q, int N_k, int d, int causal, int diag, float scale,
                   int variant, int num_splits, void* o_parts, float* lse_parts, void* stream,
                   bool dry_run = false) {
  if (B <= 0 || H <= 0 || H_kv <= 0 || H % H_kv != 0 || N_q < 0 || N_k < 0)
    return FA2_ERR_BAD_SHAPE;
  if (diag < -(1 << 30) || diag > (1 << 30)) return FA2_ERR_BAD_SHAPE;
  if (N_q == 0) return fwd_head_dim(d) ? FA2_OK : FA2_ERR_UNSUPPORTED_HEADDIM;
  if (N_k == 0) k = v = q;   // never read: every row gets O = 0, LSE = -inf
  const Variant* var = nullptr;
  int st = check_common(q, k, v, o, lse, d, scale, variant, &var);
  if (st != FA2_OK) return st;
  const long long tr = ((long long)N_q + var->br - 1) / var->br;
  const long long nbh = (long long)B * H;
  const long long wg = tr * nbh;
  // Element offsets are 64-bit in the kernel; the grid and row indices must fit 31 bits.
  if (wg > 0x7fffffffLL || nbh * (long long)N_q > 0x7fffffffLL ||
      (long long)B * H_kv * (long long)N_k > 0x7fffffffLL || (long long)N_q + N_k + 1024 > 0x7fffffffLL)
    return FA2_ERR_TOO_LARGE;
  // A causal offset beyond N_k already allows every key and one below -N_q none, so clamping
  // to [-N_q, N_k] changes no mask and keeps the kernel's 32-bit index sums in range.
  diag = diag > N_k ? N_k : (diag < -N_q ? -N_q : diag);
  int split_len = N_k, ns = 1;
  if (num_splits > 1 && N_k > 0) {
    if (!o_parts || !lse_parts) return FA2_ERR_NULL_PTR;
    if (!aligned(o_parts, 16) || !aligned(lse_parts, 4)) return FA2_ERR_MISALIGNED;
    if (num_splits > 65535) return FA2_ERR_TOO_LARGE;
    split_pieces(N_k, num_splits, var->bc, &split_len, &ns);
  }
  Params p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (uint16_t*)(ns > 1 ? o_parts : o);
  p.lse = ns > 1 ? lse_parts : lse;
  p.cu_seqlens = nullptr;
  p.nb = B;
  p.dg = d;
  p.H = H;
  p.Hkv = H_kv;
  p.g = H / H_kv;
  p.N = N_q;
  p.Nk = N_k;
  p.diag = diag;
  p.split_len = split_len;
  p.part_rows = ns > 1 ? nbh * N_q : 0;
  p.T = N_q;
  p.tr = (int)tr;
  p.heads_per_xcd = heads_per_xcd(nbh);
  fill_scale(p, scale);
  if (dry_run) return FA2_OK;
  st = launch(*var, false, causal != 0, p, (int)wg, stream, ns);
  if (st != FA2_OK || ns == 1) return st;
  return fa2_lse_merge(o_parts, lse_parts, ns, nbh * N_q, d, o, lse, stream);
}

}  // namespace

// Static scratch of fa2_fwd_splitkv_noalloc: the per-piece partial O and LSE live here instead
// of in caller workspace. Every device the library runs on holds its own copy until the
// process ends. Host code must never pass the array's name to a kernel (on the host it is a
// stand-in, not a device address): the device address comes from hipGetSymbolAddress, once
// per device, and is kept in scratch_ptr below.
static __device__ __align__(256) unsigned char scratch[FA2_STATIC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex scratch_mu;
void* scratch_ptr[kMaxDevices];   // device address of `scratch` on each device, once looked up

// The current device's copy of `scratch` (looked up on the first call on that device, with
// that device current).
int current_scratch(void** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FA2_ERR_NO_DEVICE;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return FA2_ERR_NO_DEVICE;
    scratch_ptr[dev] = ptr;
  }
  *out = scratch_ptr[dev];
  return FA2_OK;
}

}  // namespace

extern "C" {

int fa2_abi_version(void) { return FA2_ABI_VERSION; }

int fa2_num_variants(int d) {
  int count = 0;
  if (fwd_head_dim(d)) variants_for(padded_dim(d), &count);
  return count;
}

const char* fa2_variant_name(int d, int variant) {
  int count = 0;
  const Variant* vs = fwd_head_dim(d) ? variants_for(padded_dim(d), &count) : nullptr;
  if (!vs || variant < 0 || variant >= count) return "";
  return vs[variant].name;
}

int fa2_fwd_varlen_default_variant(int d) { return default_varlen_variant(d); }

const char* fa2_status_str(int status) {
  switch (status) {
    case FA2_OK: return "ok";
    case FA2_ERR_NULL_PTR: return "a required pointer is NULL";
    case FA2_ERR_BAD_SHAPE: return "bad shape (B, H must be > 0, N >= 0; varlen sizes consistent)";
    case FA2_ERR_UNSUPPORTED_HEADDIM:
      return "unsupported head dimension (a multiple of 8 from 8 to 256, forward and backward)";
    case FA2_ERR_MISALIGNED: return "misaligned pointer (q/k/v/o need 16 B, lse 4 B)";
    case FA2_ERR_BAD_SCALE: return "scale is not finite";
    case FA2_ERR_NO_DEVICE: return "no usable HIP device";
    case FA2_ERR_LAUNCH: return "kernel launch failed";
    case FA2_ERR_BAD_VARIANT: return "kernel variant out of range";
    case FA2_ERR_TOO_LARGE: return "problem too large (grid or index overflow)";
    case FA2_ERR_SCRATCH_TOO_SMALL:
      return "split-KV partials exceed the library's static scratch (FA2_STATIC_SCRATCH_BYTES per device)";
    default: return "unknown status";
  }
}

int fa2_fwd_geometry(int B, int H, int N, int d, int causal, int variant, int* num_workgroups,
                     int* block_rows, int* block_cols, int* lds_bytes) {
  (void)causal;
  if (B <= 0 || H <= 0 || N < 0) return FA2_ERR_BAD_SHAPE;
  int count = 0;
  const Variant* vs = fwd_head_dim(d) ? variants_for(padded_dim(d), &count) : nullptr;
  if (!vs) return FA2_ERR_UNSUPPORTED_HEADDIM;
  if (variant < 0 || variant >= count) return FA2_ERR_BAD_VARIANT;
  const Variant& var = vs[variant];
  const long long tr = ((long long)N + var.br - 1) / var.br;
  const long long wg = tr * (long long)B * (long long)H;
  if (wg > 0x7fffffffLL) return FA2_ERR_TOO_LARGE;
  if (num_workgroups) *num_workgroups = (int)wg;
  if (block_rows) *block_rows = var.br;
  if (block_cols) *block_cols = var.bc;
  if (lds_bytes) *lds_bytes = var.lds;
  return FA2_OK;
}

int fa2_fwd_chunk(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                  int H_kv, int N_q, int N_k, int d, int causal, int diag, float scale, int variant,
                  void* stream) {
  return fwd_chunk_impl(q, k, v, o, lse, B, H, H_kv, N_q, N_k, d, causal, diag, scale, variant, 1,
                        nullptr, nullptr, stream);
}

int fa2_fwd_splitkv(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                    int H_kv, int N_q, int N_k, int d, int causal, int diag, float scale,
                    int num_splits, void* o_parts, float* lse_parts, int variant, void* stream) {
  if (num_splits < 1) return FA2_ERR_BAD_SHAPE;
  return fwd_chunk_impl(q, k, v, o, lse, B, H, H_kv, N_q, N_k, d, causal, diag, scale, variant,
                        num_splits, o_parts, lse_parts, stream);
}

int fa2_fwd_splitkv_noalloc(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                            int H, int H_kv, int N_q, int N_k, int d, int causal, int diag, float scale,
                            int num_splits, int variant, void* stream) {
  if (num_splits < 1) return FA2_ERR_BAD_SHAPE;
  // Every argument is validated before any HIP call; the workspace stand-ins (o, lse) only
  // have to be non-null and aligned for this dry run.
  const int st0 = fwd_chunk_impl(q, k, v, o, lse, B, H, H_kv, N_q, N_k, d, causal, diag, scale, variant,
                                 num_splits, o, lse, stream, true);
  if (st0 != FA2_OK || N_q == 0) return st0;
  int count = 0;
  const Variant* vs = variants_for(padded_dim(d), &count);
  int split_len = N_k, ns = 1;
  split_pieces(N_k, num_splits, vs[variant].bc, &split_len, &ns);
  if (ns == 1)   // one piece (or no keys): the plain chunk call, no scratch
    return fwd_chunk_impl(q, k, v, o, lse, B, H, H_kv, N_q, N_k, d, causal, diag, scale, variant, 1,
                          nullptr, nullptr, stream);
  // Partial O [ns, rows, d] bf16, then partial LSE [ns, rows] fp32 at a 256-byte boundary.
  const unsigned long long rows = (unsigned long long)B * (unsigned long long)H * (unsigned long long)N_q;
  const unsigned long long obytes = ((unsigned long long)ns * rows * 2ull * (unsigned long long)d + 255ull) & ~255ull;
  const unsigned long long need = obytes + (unsigned long long)ns * rows * 4ull;
  if (need > (unsigned long long)FA2_STATIC_SCRATCH_BYTES) return FA2_ERR_SCRATCH_TOO_SMALL;
  void* base = nullptr;
  const int st = current_scratch(&base);
  if (st != FA2_OK) return st;
  unsigned char* b = (unsigned char*)base;
  return fwd_chunk_impl(q, k, v, o, lse, B, H, H_kv, N_q, N_k, d, causal, diag, scale, variant,
                        num_splits, b, (float*)(b + obytes), stream);
}

int fa2_fwd_gqa(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
                int H_kv, int N, int d, int causal, float scale, int variant, void* stream) {
  return fa2_fwd_chunk(q, k, v, o, lse, B, H, H_kv, N, N, d, causal, 0, scale, variant, stream);
}

int fa2_fwd_variant(const void* q, const void* k, const void* v, void* o, float* lse, int B,
                    int H, int N, int d, int causal, float scale, int variant, void* stream) {
  return fa2_fwd_gqa(q, k, v, o, lse, B, H, H, N, d, causal, scale, variant, stream);
}

int fa2_fwd(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H,
            int N, int d, int causal, float scale, void* stream) {
  return fa2_fwd_gqa(q, k, v, o, lse, B, H, H, N, d, causal, scale, 0, stream);
}

int fa2_fwd_varlen_gqa(const void* q, const void* k, const void* v, void* o, float* lse,
                       const int* cu_seqlens, int num_seqs, int max_seqlen, int total_tokens,
                       int H, int H_kv, int d, int causal, float scale, int variant,
                       void* stream) {
  if (H <= 0 || H_kv <= 0 || H % H_kv != 0 || num_seqs < 0 || max_seqlen < 0 ||
      total_tokens < 0)
    return FA2_ERR_BAD_SHAPE;
  if (num_seqs == 0 || total_tokens == 0 || max_seqlen == 0)
    return fwd_head_dim(d) ? FA2_OK : FA2_ERR_UNSUPPORTED_HEADDIM;
  if (!cu_seqlens) return FA2_ERR_NULL_PTR;
  if (!aligned(cu_seqlens, 4)) return FA2_ERR_MISALIGNED;
  const Variant* var = nullptr;
  int st = check_common(q, k, v, o, lse, d, scale, variant, &var);
  if (st != FA2_OK) return st;
  const long long tr = ((long long)max_seqlen + var->br - 1) / var->br;
  const long long nbh = (long long)num_seqs * H;
  const long long wg = tr * nbh;
  if (wg > 0x7fffffffLL || (long long)H * total_tokens > 0x7fffffffLL) return FA2_ERR_TOO_LARGE;
  Params p;
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (uint16_t*)o;
  p.lse = lse;
  p.cu_seqlens = cu_seqlens;
  p.nb = num_seqs;
  p.dg = d;
  p.H = H;
  p.Hkv = H_kv;
  p.g = H / H_kv;
  p.N = max_seqlen;
  p.Nk = max_seqlen;
  p.diag = 0;
  p.split_len = max_seqlen;
  p.part_rows = 0;
  p.T = total_tokens;
  p.tr = (int)tr;
  // Varlen: the plain heaviest-first order over all (sequence, head) pairs. Per-XCD pair
  // ranges leave the XCDs with unequal shares when sequence lengths differ (measured 10%
  // slower on a 16-sequence batch of 128..4096 tokens).
  p.heads_per_xcd = 0;
  fill_scale(p, scale);
  return launch(*var, true, causal != 0, p, (int)wg, stream);
}

int fa2_fwd_varlen_variant(const void* q, const void* k, const void* v, void* o, float* lse,
                           const int* cu_seqlens, int num_seqs, int max_seqlen,
                           int total_tokens, int H, int d, int causal, float scale, int variant,
                           void* stream) {
  return fa2_fwd_varlen_gqa(q, k, v, o, lse, cu_seqlens, num_seqs, max_seqlen, total_tokens, H,
                            H, d, causal, scale, variant, stream);
}

int fa2_fwd_varlen(const void* q, const void* k, const void* v, void* o, float* lse,
                   const int* cu_seqlens, int num_seqs, int max_seqlen, int total_tokens, int H,
                   int d, int causal, float scale, void* stream) {
  return fa2_fwd_varlen_gqa(q, k, v, o, lse, cu_seqlens, num_seqs, max_seqlen, total_tokens, H,
                            H, d, causal, scale, default_varlen_variant(d), stream);
}

}  // extern "C"
