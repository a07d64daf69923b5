// fa2_bwd.hip — gfx950 (CDNA4) backward kernels for exact softmax attention, and their C ABI
// (declared in include/fa2.h).
//
// Page abbreviations used below:
//   [CHL] "FlashAttention 2: Faster Attention with Better Parallelism and Work Partitioning",
//         reading notes at papers.chlience.com
//   [PGU] "FlashAttention-2: Faster Attention with Better Parallelism and Work Partitioning",
//         paper-graph-ui summary
//
// The backward of O = softmax(scale·QK^T) V, given dO, the forward's O and its logsumexp L,
// recomputes the probabilities from L instead of storing them ([CHL] 5.2, 5.3; [PGU] 3.4,
// "The Backward Pass: Simpler Statistics, Same Structure"):
//     P   = exp(scale·QK^T - L)            (0 where the causal mask removes a key)
//     D   = rowsum(dO ∘ O)
//     dV  = P^T dO
//     dP  = dO V^T
//     dS  = P ∘ (dP - D)
//     dQ  = scale · dS K
//     dK  = scale · dS^T Q
// (the pages write dQ = dS K and dK = dS^T Q for an unscaled score; with S = scale·QK^T the
// chain rule adds the factor scale). Grouped-query attention sums dK and dV over the query
// heads that share a key/value head ([CHL] 5.6).
//
// Work split. The pages' single kernel walks key/value column blocks in the outer loop and
// merges dQ across column blocks with atomic adds in HBM ([CHL] 5.4; [PGU] 3.4, "Backward
// pass parallelization"). Here the work is split over two kernels instead, which needs no
// atomics and gives bitwise-reproducible gradients:
//   fa2_bwd_dq_kernel    rows outer (one workgroup = 128 query rows, 32 per wave), key/value
//                        tiles inner: S, dP, dS, then dQ += dS K. It also writes D.
//   fa2_bwd_dkdv_kernel  columns outer (one workgroup = keys of one key/value head, 32 per
//                        wave), query tiles of every query head of the group inner: S, dP,
//                        dS, then dV += P^T dO and dK += dS^T Q.
// S and dP are computed in both (7 matrix products instead of the pages' 5).
//
// Layouts. The dQ kernel computes S^T = K Q^T and dP^T = V dO^T so that a lane owns one query
// (its statistics L and D are per lane), exactly as the forward. The dK/dV kernel computes
// S = Q K^T and dP = dO V^T so that a lane owns one key; P and dS then sit in registers in the
// B-operand layout of dV^T = dO^T P and dK^T = Q^T dS, whose A operands (dO^T, Q^T) are
// gathered from row-major tiles in LDS by transposed reads. Tiles that are read both by rows
// and transposed use a swizzle that keeps both read patterns free of bank conflicts.

#include <hip/hip_runtime.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "fa2.h"
#include "fa2_dev.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

struct BwdParams {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const float* lse;
  const uint16_t* dout;
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  float* delta;           // D = rowsum(dO ∘ O), fp32, laid out like lse
  const int* cu_seqlens;  // varlen only
  int nb;                 // batch size, or number of sequences (varlen)
  int dg;                 // head dimension of the tensors (multiple of 8, <= D; see below)
  int H;                  // query heads
  int Hkv;                // key/value heads
  int g;                  // H / Hkv
  int N;                  // sequence length, or max_seqlen (varlen)
  int T;                  // tokens per head plane: N, or total_tokens (varlen)
  int nblk;               // 128-row (dQ) or 128-key (dK/dV) blocks per sequence
  int heads_per_xcd;      // > 0: XCD-aware workgroup order
  int hsplit;             // dK/dV: workgroups per (key/value head, key block), each taking
                          // g / hsplit query heads of the group; 1 = the whole group
  float* kv_ws;           // hsplit > 1: fp32 partial dK, dV per split, [hsplit][2][ws_slab]
  long long ws_slab;      // elements of one partial (key/value rows x dg)
  float c;                // |scale| * log2(e), at least 1e-30
  float scale;            // the signed softmax scale
  uint32_t qflip;         // 0x80008000 negates Q in the score products (scale < 0), else 0
};

// Row swizzle of a bf16 tile in LDS (16-byte chunk index XOR per row), chosen so that both
// access patterns used on one tile are free of bank conflicts: 16-byte row reads by 16
// consecutive rows at one logical chunk, and transposed 8-byte reads of 4 consecutive rows
// (starting at a multiple of 4) by 4 consecutive chunks. Period 16 in the row index.
// D = 256 rows (512 bytes, two bank sweeps) use the D = 128 pattern on the low four bits of
// the chunk index. Every swizzle value is below 16, so logical chunk c + 16 of a row lies 256
// bytes after chunk c: read offsets are kept for chunks 0..15 and the rest reached through
// the instructions' immediate offset (roff/toff below).
template <int D>
__device__ __forceinline__ int dswz(int row) {
  return D >= 128 ? (((row & 3) << 2) | ((row >> 2) & 3))
                  : ((((row >> 1) & 1) << 2) | ((row >> 2) & 3));
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Work item id -> (pair index in [0, npairs), block index). As in the forward: workgroup id
// goes to XCD id % 8 and, when npairs % 8 == 0, each XCD owns a contiguous set of pairs.
// Causal launches start with the heaviest blocks: HEAVY_HIGH puts the largest block index
// first (query blocks of the dQ kernel), otherwise the smallest (key blocks of dK/dV).
template <bool CAUSAL, bool HEAVY_HIGH>
__device__ __forceinline__ void decode_bwd(int id, int npairs, int nblk, int hpx, int& pair, int& blk) {
  if (hpx > 0) {
    const int x = id & 7, slot = id >> 3;
    int hl;
    if (CAUSAL) {
      const int r = slot / hpx;
      blk = HEAVY_HIGH ? nblk - 1 - r : r;
      hl = slot - r * hpx;
    } else {
      hl = slot / nblk;
      blk = slot - hl * nblk;
    }
    pair = x * hpx + hl;
  } else {
    const int r = id / npairs;
    blk = (CAUSAL && !HEAVY_HIGH) ? r : nblk - 1 - r;
    pair = id - r * npairs;
  }
}

// Token range of sequence bi: [tok0, tok0 + len) of each head plane.
template <bool VARLEN>
__device__ __forceinline__ void seq_range(const BwdParams& p, int bi, int& tok0, int& len) {
  if (VARLEN) {
    int a = p.cu_seqlens[bi];
    int e = p.cu_seqlens[bi + 1];
    a = min(max(a, 0), p.T);
    e = min(max(e, a), p.T);
    tok0 = a;
    len = e - a;
  } else {
    tok0 = 0;
    len = p.N;
  }
}

// First element (row index into [.., T, D] arrays) of the plane of query head h / key-value
// head hk of batch (or sequence) bi.
template <bool VARLEN>
__device__ __forceinline__ size_t q_plane(const BwdParams& p, int bi, int h) {
  return VARLEN ? (size_t)h * (size_t)p.T : ((size_t)bi * p.H + h) * (size_t)p.N;
}
template <bool VARLEN>
__device__ __forceinline__ size_t kv_plane(const BwdParams& p, int bi, int hk) {
  return VARLEN ? (size_t)hk * (size_t)p.T : ((size_t)bi * p.Hkv + hk) * (size_t)p.N;
}

// ---- dQ kernel -------------------------------------------------------------------------

template <int D, int BC, int NW = 4>
struct DqTile {
  static constexpr int WAVES = NW;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BR = 32 * WAVES;
  static constexpr int ROWB = 2 * D;
  static constexpr int TILEB = BC * ROWB;           // one K (or V) tile
  static constexpr int STAGEB = 2 * TILEB;          // K tile then V tile
  static constexpr int LDS_BYTES = 2 * STAGEB;
  static constexpr int DMA_PER_WAVE = TILEB / 1024 / WAVES;
  static constexpr int NKB = BC / 32;
  static constexpr int NKC = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int NPC = BC / 16;
  static_assert(D == 64 || D == 128 || D == 256, "head dim");
  static_assert(BC % 32 == 0 && DMA_PER_WAVE >= 1 && TILEB % (1024 * WAVES) == 0, "tile shape");
};

// LA: the K and V row fragments of S^T and dP^T are read LA fragments ahead of the MFMAs
// that use them (0: the compiler's order, which issues each read one MFMA before its use).
template <int D, int BC, bool CAUSAL, bool VARLEN, int NW, int LA_, bool PERSIST>
__device__ __forceinline__ void bwd_dq_block(const BwdParams& p, int id) {
  using TL = DqTile<D, BC, NW>;
  __shared__ __attribute__((aligned(1024))) unsigned char lds0[TL::STAGEB];
  __shared__ __attribute__((aligned(1024))) unsigned char lds1[TL::STAGEB];

  int tid = threadIdx.x;
  // In the persistent kernels this block is one iteration of a loop over blocks. An opaque
  // copy of the thread id keeps the compiler from hoisting the lane-derived offsets out of
  // that loop, where they would stay live, and spill, across every block.
  if constexpr (PERSIST) asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  int bh, i;
  decode_bwd<CAUSAL, true>(id, p.nb * p.H, p.nblk, p.heads_per_xcd, bh, i);
  const int bi = bh / p.H;
  const int h = bh - bi * p.H;
  int tok0, seq_len;
  seq_range<VARLEN>(p, bi, tok0, seq_len);
  const int q0 = i * TL::BR;
  if (q0 >= seq_len) return;
  const size_t row0 = q_plane<VARLEN>(p, bi, h) + (size_t)tok0;
  const size_t kvrow0 = kv_plane<VARLEN>(p, bi, h / p.g) + (size_t)tok0;
  const int dg = p.dg;          // row pitch of every tensor, in elements
  const int growb = 2 * dg;
  const unsigned char* kh = (const unsigned char*)(p.k + kvrow0 * dg);
  const unsigned char* vh = (const unsigned char*)(p.v + kvrow0 * dg);
  const int kv_end = CAUSAL ? min(seq_len, q0 + TL::BR) : seq_len;
  const int nt = (kv_end + BC - 1) / BC;

  // K/V staging (direct global -> LDS), both tiles with the dual-pattern swizzle.
  int drow_[TL::DMA_PER_WAVE];
  uint32_t doff[TL::DMA_PER_WAVE];
#pragma unroll
  for (int d = 0; d < TL::DMA_PER_WAVE; ++d) {
    const int b = wave * TL::DMA_PER_WAVE + d;
    const int o = b * 1024 + lane * 16;
    const int r = o / TL::ROWB;
    const int pch = (o % TL::ROWB) / 16;
    drow_[d] = r;
    doff[d] = r * growb + (((pch ^ dswz<D>(r)) % (dg / 8)) * 16);
  }
  auto dma_tile = [&](int j, unsigned char* stage) {
    const int key0 = j * BC;
    const unsigned char* kt = kh + (size_t)key0 * growb;
    const unsigned char* vt = vh + (size_t)key0 * growb;
    const uint32_t ks_a = lds_addr(stage) + wave * TL::DMA_PER_WAVE * 1024;
    const uint32_t vs_a = lds_addr(stage + TL::TILEB) + wave * TL::DMA_PER_WAVE * 1024;
    const int last = seq_len - 1 - key0;   // rows past the end re-read the last valid row
#pragma unroll
    for (int d = 0; d < TL::DMA_PER_WAVE; ++d) {
      const uint32_t back = (uint32_t)(drow_[d] - min(drow_[d], last)) * growb;
      dma16(kt, doff[d] - back, ks_a + d * 1024);
      dma16(vt, doff[d] - back, vs_a + d * 1024);
    }
  };

  dma_tile(0, lds0);

  // This lane's query: Q^T and dO^T as B fragments, L in base 2, and D = rowsum(dO ∘ O)
  // (each 32-lane half holds 8 of every 16 head-dimension values). Issued after tile 0's
  // K/V loads and without branches (see col_mask); a row past the end reads row seq_len - 1,
  // whose values only reach that row's dQ and D, which are never written.
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;
  const bool valid = qrow < seq_len;
  const size_t rrow = row0 + (size_t)min(qrow, seq_len - 1);
  bf16x8 qf[TL::NKC], df[TL::NKC];
  float dot = 0.f;
  {
    u32x4 tq[TL::NKC], td[TL::NKC], to[TL::NKC];
#pragma unroll
    for (int kc = 0; kc < TL::NKC; ++kc) {
      const int col = kc * 16 + hl * 8;
      const size_t off = rrow * dg + (col < dg ? col : 0);
      tq[kc] = *(const u32x4*)(p.q + off);
      td[kc] = *(const u32x4*)(p.dout + off);
      to[kc] = *(const u32x4*)(p.o + off);
    }
#pragma unroll
    for (int kc = 0; kc < TL::NKC; ++kc) {
      const uint32_t m = col_mask(kc * 16 + hl * 8, dg);
      const u32x4 d4 = td[kc] & m, o4 = to[kc] & m;
#pragma unroll
      for (int e = 0; e < 4; ++e)
        dot += bf16_lo(d4[e]) * bf16_lo(o4[e]) + bf16_hi(d4[e]) * bf16_hi(o4[e]);
      qf[kc] = as_bf16x8((tq[kc] & m) ^ p.qflip);
      df[kc] = as_bf16x8(d4);
    }
  }
  const float drow = halves_sum(dot);
  const float l2 = p.lse[rrow] * kLog2e;
  if (valid && hl == 0) p.delta[row0 + (size_t)qrow] = drow;

  // Row reads (A operands of S^T and dP^T): row kb*32 + l32, logical chunk 2kc + hl.
  constexpr int NRA = TL::NKC < 8 ? TL::NKC : 8;
  int raddr[NRA];
#pragma unroll
  for (int kc = 0; kc < NRA; ++kc)
    raddr[kc] = l32 * TL::ROWB + (((2 * kc + hl) ^ dswz<D>(l32)) * 16);
  auto roff = [&](int kc) { return raddr[kc & 7] + (kc >> 3) * 256; };
  // Transposed reads of K (A operand K^T of dQ^T): rows 16c + 4hl + (lane%16)/4 (low half of
  // the fragment) and the same + 8 (high half), columns 32db + 16((lane/16)%2) + 4(lane%4).
  const int tr0 = 4 * hl + ((lane & 15) >> 2);
  constexpr int NTA = TL::NDB < 4 ? TL::NDB : 4;
  int taddr_lo[NTA], taddr_hi[NTA];
#pragma unroll
  for (int db = 0; db < NTA; ++db) {
    const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    taddr_lo[db] = tr0 * TL::ROWB + (((col >> 3) ^ dswz<D>(tr0)) * 16) + (col & 7) * 2;
    taddr_hi[db] = (tr0 + 8) * TL::ROWB + (((col >> 3) ^ dswz<D>(tr0 + 8)) * 16) + (col & 7) * 2;
  }
  auto toff_lo = [&](int db) { return taddr_lo[db & 3] + (db >> 2) * 256; };
  auto toff_hi = [&](int db) { return taddr_hi[db & 3] + (db >> 2) * 256; };

  f32x16 dqacc[TL::NDB];
#pragma unroll
  for (int db = 0; db < TL::NDB; ++db) dqacc[db] = (f32x16){};

  auto compute_tile = [&](int j, const unsigned char* stage) {
    const int key0 = j * BC;
    if ((CAUSAL && key0 > qw0 + 31) || qw0 >= seq_len) return;
    f32x16 s[TL::NKB], dp[TL::NKB];
#pragma unroll
    for (int kb = 0; kb < TL::NKB; ++kb) {
      s[kb] = (f32x16){};
      dp[kb] = (f32x16){};
    }
    {
      // Fragment f = kb*NKC + kc: its K and V rows are read LA fragments ahead of the two
      // MFMAs that use them (a ring of LA register pairs; the fences keep the order).
      constexpr int NF = TL::NKB * TL::NKC;
      constexpr int LA = LA_ > 0 ? (LA_ < NF ? LA_ : NF) : 1;
      bf16x8 kr[LA], vr[LA];
      auto rd = [&](int f) {
        const int kb = f / TL::NKC, kc = f % TL::NKC;
        kr[f % LA] = *(const bf16x8*)(stage + kb * 32 * TL::ROWB + roff(kc));
        vr[f % LA] = *(const bf16x8*)(stage + TL::TILEB + kb * 32 * TL::ROWB + roff(kc));
      };
#pragma unroll
      for (int f = 0; f < LA; ++f) rd(f);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int kb = f / TL::NKC, kc = f % TL::NKC;
        if constexpr (LA_ > 0) __builtin_amdgcn_sched_barrier(0);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kr[f % LA], qf[kc], s[kb], 0, 0, 0);
        dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vr[f % LA], df[kc], dp[kb], 0, 0, 0);
        if (f + LA < NF) rd(f + LA);
      }
      if constexpr (LA_ > 0) __builtin_amdgcn_sched_barrier(0);
    }
    // Causal and ragged masks (key > query, key >= length), as in the forward.
    if ((CAUSAL && key0 + BC - 1 > qw0) || key0 + BC > seq_len) {
      int thr = seq_len - 1 - key0 - 4 * hl;
      if (CAUSAL) thr = min(thr, qrow - key0 - 4 * hl);
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
    // P = 2^(S·c - L2), dS = P ∘ (dP - D), packed as the B operand of dQ^T (key order of a
    // contraction step c as in the forward's P~).
    u32x4 dsw[TL::NPC];
#pragma unroll
    for (int c = 0; c < TL::NPC; ++c) {
      const int kb = c >> 1, r0 = (c & 1) * 8;
      float e[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const float pv = __builtin_amdgcn_exp2f(fmaf(s[kb][r0 + u], p.c, -l2));
        e[u] = pv * (dp[kb][r0 + u] - drow);
      }
      dsw[c] = (u32x4){pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]),
                       pack_bf16x2(e[4], e[5]), pack_bf16x2(e[6], e[7])};
    }
    // dQ^T += K^T dS^T, fragment f = c*NDB + db, its K^T fragment read LA fragments ahead (the
    // fences let VALU and SALU work cross, not MFMAs or LDS reads).
    {
      constexpr int NF = TL::NPC * TL::NDB;
      constexpr int LA = LA_ > 0 ? (LA_ < NF ? LA_ : NF) : 1;
      bf16x8 ta[LA];
      auto rd = [&](int f) {
        const int c = f / TL::NDB, db = f % TL::NDB;
        const unsigned char* base = stage + 16 * c * TL::ROWB;
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, base + toff_lo(db)));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, base + toff_hi(db)));
        ta[f % LA] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
#pragma unroll
      for (int f = 0; f < LA; ++f) rd(f);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int c = f / TL::NDB, db = f % TL::NDB;
        if constexpr (LA_ > 0) __builtin_amdgcn_sched_barrier(0x406);
        dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta[f % LA], as_bf16x8(dsw[c]), dqacc[db], 0, 0, 0);
        if (f + LA < NF) rd(f + LA);
      }
      if constexpr (LA_ > 0) __builtin_amdgcn_sched_barrier(0x406);
    }
  };

  auto iteration = [&](int j, unsigned char* cur, unsigned char* nxt) {
    if (j + 1 < nt) dma_tile(j + 1, nxt);
    compute_tile(j, cur);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // tile 0, issued before the row loads
  __syncthreads();
  for (int j = 0; j < nt; j += 2) {
    iteration(j, lds0, lds1);
    if (j + 1 < nt) iteration(j + 1, lds1, lds0);
  }

  if (valid) {
    uint16_t* out = p.dq + (row0 + (size_t)qrow) * dg;
#pragma unroll
    for (int db = 0; db < TL::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 w = {pack_bf16x2(dqacc[db][4 * g + 0] * p.scale, dqacc[db][4 * g + 1] * p.scale),
                   pack_bf16x2(dqacc[db][4 * g + 2] * p.scale, dqacc[db][4 * g + 3] * p.scale)};
        if (db * 32 + 8 * g + 4 * hl < dg) *(u32x2*)(out + db * 32 + 8 * g + 4 * hl) = w;
      }
  }
}

// One workgroup per 128-row block; or, in the persistent form that varlen calls take at
// d = 128 and 256, as many workgroups as the CUs hold, taking blocks from a work queue.
template <int D, int BC, bool CAUSAL, bool VARLEN, int NW, int OCC, int LA_>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(OCC, OCC)))
void fa2_bwd_dq_kernel(BwdParams p) {
  bwd_dq_block<D, BC, CAUSAL, VARLEN, NW, LA_, false>(p, (int)blockIdx.x);
}
template <int D, int BC, bool CAUSAL, bool VARLEN, int NW, int OCC, int LA_>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(OCC, OCC)))
void fa2_bwd_dq_kernel_persist(BwdParams p, unsigned int* ctr, int total) {
  run_work_queue(ctr, 1, total, [&](int id) { bwd_dq_block<D, BC, CAUSAL, VARLEN, NW, LA_, true>(p, id); });
}

// ---- dK/dV kernel ----------------------------------------------------------------------

template <int D, int BQ, int NW = 4>
struct DkvTile {
  static constexpr int WAVES = NW;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int BK = 32 * WAVES;             // keys per workgroup
  static constexpr int ROWB = 2 * D;
  static constexpr int TILEB = BQ * ROWB;           // one Q (or dO) tile
  static constexpr int VECB = 256;                  // one L (or D) vector: 64 fp32 loaded, first BQ used
  static constexpr int STAGEB = 2 * TILEB + 2 * VECB;
  static constexpr int LDS_BYTES = 2 * STAGEB;
  static constexpr int DMA_PER_WAVE = TILEB / 1024 / WAVES;
  static constexpr int NQB = BQ / 32;               // 32-query blocks per tile
  static constexpr int NKC = D / 16;
  static constexpr int NDB = D / 32;
  static constexpr int NPC = BQ / 16;
  static_assert(D == 64 || D == 128 || D == 256, "head dim");
  static_assert(BQ == 64 || BQ == 32, "statistics vectors are one 256-byte direct load");
  static_assert(DMA_PER_WAVE >= 1 && TILEB % (1024 * WAVES) == 0, "tile shape");
};

// KLDS: the wave's K rows are kept in LDS (stored once, in the swizzled layout of the Q row
// reads) instead of 32 registers, which lets d = 128 run two waves per SIMD. LA as in the dQ
// kernel, for the Q and dO (and K) row fragments of S and dP.
template <int D, int BQ, bool CAUSAL, bool VARLEN, int NW, bool KLDS, int LA_, int LA_ACC, bool PERSIST>
__device__ __forceinline__ void bwd_dkdv_block(const BwdParams& p, int id) {
  using TL = DkvTile<D, BQ, NW>;
  __shared__ __attribute__((aligned(1024))) unsigned char lds0[TL::STAGEB];
  __shared__ __attribute__((aligned(1024))) unsigned char lds1[TL::STAGEB];
  __shared__ __attribute__((aligned(1024))) unsigned char kst[KLDS ? TL::BK * TL::ROWB : 16];

  int tid = threadIdx.x;
  // In the persistent kernels this block is one iteration of a loop over blocks. An opaque
  // copy of the thread id keeps the compiler from hoisting the lane-derived offsets out of
  // that loop, where they would stay live, and spill, across every block.
  if constexpr (PERSIST) asm volatile("" : "+v"(tid));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hl = lane >> 5;

  // Work item: (batch or sequence, key/value head, query-head split) x key block. The splits
  // of one key/value head are adjacent, so they share an XCD and the heaviest-first order.
  int bks, jb;
  decode_bwd<CAUSAL, false>(id, p.nb * p.Hkv * p.hsplit, p.nblk, p.heads_per_xcd, bks, jb);
  const int bk = bks / p.hsplit;
  const int sp = bks - bk * p.hsplit;   // this split's query heads: [sp * gs, sp * gs + gs)
  const int gs = p.g / p.hsplit;
  const int bi = bk / p.Hkv;
  const int hk = bk - bi * p.Hkv;
  int tok0, seq_len;
  seq_range<VARLEN>(p, bi, tok0, seq_len);
  const int k0 = jb * TL::BK;
  if (k0 >= seq_len) return;
  const size_t kvrow0 = kv_plane<VARLEN>(p, bi, hk) + (size_t)tok0;
  const int dg = p.dg;          // row pitch of every tensor, in elements
  const int growb = 2 * dg;

  // This wave's 32 keys as B fragments of S = Q K^T and dP = dO V^T (key kw0 + l32).
  const int kw0 = k0 + wave * 32;
  const int krow = kw0 + l32;
  const bool kvalid = krow < seq_len;
  bf16x8 kf[TL::NKC], vf[TL::NKC];
#pragma unroll
  for (int kc = 0; kc < TL::NKC; ++kc) {
    u32x4 tk = {0u, 0u, 0u, 0u}, tv = tk;
    if (kvalid && kc * 16 + hl * 8 < dg) {
      const size_t off = (kvrow0 + (size_t)krow) * dg + kc * 16 + hl * 8;
      tk = *(const u32x4*)(p.k + off);
      tv = *(const u32x4*)(p.v + off);
    }
    kf[kc] = as_bf16x8(tk ^ p.qflip);
    vf[kc] = as_bf16x8(tv);
  }

  // Query tiles: causal starts at the tile holding query k0; every query head of the split.
  const int t0 = CAUSAL ? k0 / BQ : 0;
  const int ntq = (seq_len + BQ - 1) / BQ - t0;
  const int nsteps = ntq * gs;

  int drow_[TL::DMA_PER_WAVE];
  uint32_t doff[TL::DMA_PER_WAVE];
#pragma unroll
  for (int d = 0; d < TL::DMA_PER_WAVE; ++d) {
    const int b = wave * TL::DMA_PER_WAVE + d;
    const int o = b * 1024 + lane * 16;
    const int r = o / TL::ROWB;
    const int pch = (o % TL::ROWB) / 16;
    drow_[d] = r;
    doff[d] = r * growb + (((pch ^ dswz<D>(r)) % (dg / 8)) * 16);
  }
  auto step_coords = [&](int s, int& q0, size_t& qrow0) {
    const int hq = s / ntq;
    q0 = (t0 + (s - hq * ntq)) * BQ;
    qrow0 = q_plane<VARLEN>(p, bi, hk * p.g + sp * gs + hq) + (size_t)tok0;
  };
  auto dma_step = [&](int s, unsigned char* stage) {
    int q0;
    size_t qrow0;
    step_coords(s, q0, qrow0);
    const unsigned char* qt = (const unsigned char*)(p.q + (qrow0 + q0) * dg);
    const unsigned char* dt = (const unsigned char*)(p.dout + (qrow0 + q0) * dg);
    const uint32_t qs_a = lds_addr(stage) + wave * TL::DMA_PER_WAVE * 1024;
    const uint32_t ds_a = lds_addr(stage + TL::TILEB) + wave * TL::DMA_PER_WAVE * 1024;
    const int last = seq_len - 1 - q0;    // rows past the end re-read the last valid row
#pragma unroll
    for (int d = 0; d < TL::DMA_PER_WAVE; ++d) {
      const uint32_t back = (uint32_t)(drow_[d] - min(drow_[d], last)) * growb;
      dma16(qt, doff[d] - back, qs_a + d * 1024);
      dma16(dt, doff[d] - back, ds_a + d * 1024);
    }
    // Statistics of the tile's rows: L (wave 0) and D (wave 1), one dword per lane.
    if (wave < 2) {
      const float* src = (wave == 0 ? p.lse : p.delta) + qrow0 + q0;
      const uint32_t voff = (uint32_t)min(lane, last) * 4u;
      dma4(src, voff, lds_addr(stage + 2 * TL::TILEB + wave * TL::VECB));
    }
  };

  // Row reads (A operands of S and dP): row qb*32 + l32, logical chunk 2kc + hl.
  constexpr int NRA = TL::NKC < 8 ? TL::NKC : 8;
  int raddr[NRA];
#pragma unroll
  for (int kc = 0; kc < NRA; ++kc)
    raddr[kc] = l32 * TL::ROWB + (((2 * kc + hl) ^ dswz<D>(l32)) * 16);
  auto roff = [&](int kc) { return raddr[kc & 7] + (kc >> 3) * 256; };
  // K rows of this wave in LDS: row l32 of the wave's 32-row slab, chunk 2kc + hl, at the
  // same swizzled offsets as the Q row reads (the slab starts at a multiple of 32 rows, and
  // the swizzle depends on the row's low four bits only). Published by the barrier that
  // precedes the first step.
  const uint32_t kslab = (uint32_t)wave * 32u * TL::ROWB;
  if constexpr (KLDS) {
#pragma unroll
    for (int kc = 0; kc < TL::NKC; ++kc) *(bf16x8*)(kst + kslab + roff(kc)) = kf[kc];
  }
  // Transposed reads (A operands dO^T and Q^T), as K^T in the dQ kernel.
  const int tr0 = 4 * hl + ((lane & 15) >> 2);
  constexpr int NTA = TL::NDB < 4 ? TL::NDB : 4;
  int taddr_lo[NTA], taddr_hi[NTA];
#pragma unroll
  for (int db = 0; db < NTA; ++db) {
    const int col = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    taddr_lo[db] = tr0 * TL::ROWB + (((col >> 3) ^ dswz<D>(tr0)) * 16) + (col & 7) * 2;
    taddr_hi[db] = (tr0 + 8) * TL::ROWB + (((col >> 3) ^ dswz<D>(tr0 + 8)) * 16) + (col & 7) * 2;
  }
  auto toff_lo = [&](int db) { return taddr_lo[db & 3] + (db >> 2) * 256; };
  auto toff_hi = [&](int db) { return taddr_hi[db & 3] + (db >> 2) * 256; };

  f32x16 dkacc[TL::NDB], dvacc[TL::NDB];
#pragma unroll
  for (int db = 0; db < TL::NDB; ++db) {
    dkacc[db] = (f32x16){};
    dvacc[db] = (f32x16){};
  }

  auto compute_step = [&](int s_idx, const unsigned char* stage) {
    int q0;
    size_t qrow0;
    step_coords(s_idx, q0, qrow0);
    if ((CAUSAL && q0 + BQ - 1 < kw0) || kw0 >= seq_len) return;
    // S = Q K^T and dP = dO V^T: lane = key, entries r = queries 32qb + 8(r/4) + 4hl + r%4.
    f32x16 s[TL::NQB], dp[TL::NQB];
#pragma unroll
    for (int qb = 0; qb < TL::NQB; ++qb) {
      s[qb] = (f32x16){};
      dp[qb] = (f32x16){};
    }
    {
      // Fragment f = qb*NKC + kc: its Q and dO rows (and the K rows kept in LDS) are read LA
      // fragments ahead of the two MFMAs that use them.
      constexpr int NF = TL::NQB * TL::NKC;
      constexpr int LA = LA_ > 0 ? (LA_ < NF ? LA_ : NF) : 1;
      bf16x8 qr[LA], dr[LA], kr[LA];
      auto rd = [&](int f) {
        const int qb = f / TL::NKC, kc = f % TL::NKC;
        qr[f % LA] = *(const bf16x8*)(stage + qb * 32 * TL::ROWB + roff(kc));
        dr[f % LA] = *(const bf16x8*)(stage + TL::TILEB + qb * 32 * TL::ROWB + roff(kc));
        kr[f % LA] = KLDS ? *(const bf16x8*)(kst + kslab + roff(kc)) : kf[kc];
      };
#pragma unroll
      for (int f = 0; f < LA; ++f) rd(f);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int qb = f / TL::NKC, kc = f % TL::NKC;
        if constexpr (LA_ > 0) __builtin_amdgcn_sched_barrier(0);
        s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qr[f % LA], kr[f % LA], s[qb], 0, 0, 0);
        dp[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dr[f % LA], vf[kc], dp[qb], 0, 0, 0);
        if (f + LA < NF) rd(f + LA);
      }
      if constexpr (LA_ > 0) __builtin_amdgcn_sched_barrier(0);
    }
    // Masks: query < key (causal), query >= length (ragged tile). With off the entry's query
    // offset minus 4hl (a constant), dead when off < lo or off > hi.
    if ((CAUSAL && q0 < kw0 + 31) || q0 + BQ > seq_len) {
      const int lo = krow - q0 - 4 * hl;
      const int hi = seq_len - 1 - q0 - 4 * hl;
#pragma unroll
      for (int qb = 0; qb < TL::NQB; ++qb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = qb * 32 + 8 * (r >> 2) + (r & 3);
          uint32_t dead = (uint32_t)((hi - off) >> 31);
          if (CAUSAL) dead |= (uint32_t)((off - lo) >> 31);
          const uint32_t bits = __float_as_uint(s[qb][r]);
          s[qb][r] = __uint_as_float((bits & ~dead) | (0xff800000u & dead));
        }
    }
    // P and dS, packed as B operands (query order of contraction step c as the forward's
    // key order of P~).
    const unsigned char* lvec = stage + 2 * TL::TILEB;
    const unsigned char* dvec = lvec + TL::VECB;
    u32x4 pw[TL::NPC], dsw[TL::NPC];
#pragma unroll
    for (int c = 0; c < TL::NPC; ++c) {
      const int qb = c >> 1, r0 = (c & 1) * 8;
      float pe[8], de[8];
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        // queries 32qb + 8(r/4) + 4hl + 0..3 for r = r0 + 4half .. +3
        const int qo = qb * 32 + 8 * ((r0 >> 2) + half) + 4 * hl;
        const float4 lv = *(const float4*)(lvec + 4 * qo);
        const float4 dv = *(const float4*)(dvec + 4 * qo);
        const float lq[4] = {lv.x, lv.y, lv.z, lv.w};
        const float dq[4] = {dv.x, dv.y, dv.z, dv.w};
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int u = 4 * half + t;
          const float pv = __builtin_amdgcn_exp2f(fmaf(s[qb][r0 + u], p.c, -lq[t] * kLog2e));
          pe[u] = pv;
          de[u] = pv * (dp[qb][r0 + u] - dq[t]);
        }
      }
      pw[c] = (u32x4){pack_bf16x2(pe[0], pe[1]), pack_bf16x2(pe[2], pe[3]),
                      pack_bf16x2(pe[4], pe[5]), pack_bf16x2(pe[6], pe[7])};
      dsw[c] = (u32x4){pack_bf16x2(de[0], de[1]), pack_bf16x2(de[2], de[3]),
                       pack_bf16x2(de[4], de[5]), pack_bf16x2(de[6], de[7])};
    }
    // dV^T += dO^T P, dK^T += Q^T dS, fragment f = c*NDB + db: its dO^T and Q^T fragments
    // are read LA_ACC fragments ahead (fences as in the dQ kernel).
    {
      constexpr int NF = TL::NPC * TL::NDB;
      constexpr int LA = LA_ACC > 0 ? (LA_ACC < NF ? LA_ACC : NF) : 1;
      bf16x8 da[LA], qa[LA];
      auto rd = [&](int f) {
        const int c = f / TL::NDB, db = f % TL::NDB;
        const unsigned char* qbase = stage + 16 * c * TL::ROWB;
        const unsigned char* dbase = stage + TL::TILEB + 16 * c * TL::ROWB;
        const i16x4 dlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, dbase + toff_lo(db)));
        const i16x4 dhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, dbase + toff_hi(db)));
        const i16x4 qlo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, qbase + toff_lo(db)));
        const i16x4 qhi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, qbase + toff_hi(db)));
        da[f % LA] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(dlo, dhi, 0, 1, 2, 3, 4, 5, 6, 7));
        qa[f % LA] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7));
      };
#pragma unroll
      for (int f = 0; f < LA; ++f) rd(f);
#pragma unroll
      for (int f = 0; f < NF; ++f) {
        const int c = f / TL::NDB, db = f % TL::NDB;
        if constexpr (LA_ACC > 0) __builtin_amdgcn_sched_barrier(0x406);
        dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da[f % LA], as_bf16x8(pw[c]), dvacc[db], 0, 0, 0);
        dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[f % LA], as_bf16x8(dsw[c]), dkacc[db], 0, 0, 0);
        if (f + LA < NF) rd(f + LA);
      }
      if constexpr (LA_ACC > 0) __builtin_amdgcn_sched_barrier(0x406);
    }
  };

  auto iteration = [&](int st, unsigned char* cur, unsigned char* nxt) {
    if (st + 1 < nsteps) dma_step(st + 1, nxt);
    compute_step(st, cur);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
  };
  dma_step(0, lds0);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  for (int st = 0; st < nsteps; st += 2) {
    iteration(st, lds0, lds1);
    if (st + 1 < nsteps) iteration(st + 1, lds1, lds0);
  }

  if (kvalid && p.hsplit > 1) {
    // This split's share of the sums over the group: fp32 partials, added up in split order
    // by fa2_bwd_kv_reduce_kernel.
    float* kw = p.kv_ws + (size_t)sp * 2 * (size_t)p.ws_slab + (kvrow0 + (size_t)krow) * dg;
    float* vw = kw + p.ws_slab;
#pragma unroll
    for (int db = 0; db < TL::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        if (db * 32 + 8 * g + 4 * hl < dg) {
          const int c = db * 32 + 8 * g + 4 * hl;
          *(f32x4*)(kw + c) = (f32x4){dkacc[db][4 * g + 0] * p.scale, dkacc[db][4 * g + 1] * p.scale,
                                      dkacc[db][4 * g + 2] * p.scale, dkacc[db][4 * g + 3] * p.scale};
          *(f32x4*)(vw + c) = (f32x4){dvacc[db][4 * g + 0], dvacc[db][4 * g + 1],
                                      dvacc[db][4 * g + 2], dvacc[db][4 * g + 3]};
        }
  } else if (kvalid) {
    uint16_t* kout = p.dk + (kvrow0 + (size_t)krow) * dg;
    uint16_t* vout = p.dv + (kvrow0 + (size_t)krow) * dg;
#pragma unroll
    for (int db = 0; db < TL::NDB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        u32x2 wk = {pack_bf16x2(dkacc[db][4 * g + 0] * p.scale, dkacc[db][4 * g + 1] * p.scale),
                    pack_bf16x2(dkacc[db][4 * g + 2] * p.scale, dkacc[db][4 * g + 3] * p.scale)};
        u32x2 wv = {pack_bf16x2(dvacc[db][4 * g + 0], dvacc[db][4 * g + 1]),
                    pack_bf16x2(dvacc[db][4 * g + 2], dvacc[db][4 * g + 3])};
        if (db * 32 + 8 * g + 4 * hl < dg) {
          *(u32x2*)(kout + db * 32 + 8 * g + 4 * hl) = wk;
          *(u32x2*)(vout + db * 32 + 8 * g + 4 * hl) = wv;
        }
      }
  }
}

template <int D, int BQ, bool CAUSAL, bool VARLEN, int NW, int OCC, bool KLDS, int LA_, int LA_ACC>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(OCC, OCC)))
void fa2_bwd_dkdv_kernel(BwdParams p) {
  bwd_dkdv_block<D, BQ, CAUSAL, VARLEN, NW, KLDS, LA_, LA_ACC, false>(p, (int)blockIdx.x);
}
template <int D, int BQ, bool CAUSAL, bool VARLEN, int NW, int OCC, bool KLDS, int LA_, int LA_ACC>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(OCC, OCC)))
void fa2_bwd_dkdv_kernel_persist(BwdParams p, unsigned int* ctr, int total) {
  run_work_queue(ctr, 1, total,
                 [&](int id) { bwd_dkdv_block<D, BQ, CAUSAL, VARLEN, NW, KLDS, LA_, LA_ACC, true>(p, id); });
}

// Sum of the query-head splits' partial dK and dV, in split order (fixed, so the bits do not
// depend on timing), rounded to bf16 as the unsplit epilogue rounds. Thread i handles
// elements [4i, 4i + 4) of both; slab is a multiple of 8.
__global__ __launch_bounds__(256) void fa2_bwd_kv_reduce_kernel(const float* __restrict__ ws, long long slab,
                                                                int nsplit, uint16_t* __restrict__ dk,
                                                                uint16_t* __restrict__ dv) {
  const long long e = 4 * ((long long)blockIdx.x * 256 + threadIdx.x);
  if (e >= slab) return;
  f32x4 ak = *(const f32x4*)(ws + e);
  f32x4 av = *(const f32x4*)(ws + slab + e);
  for (int s = 1; s < nsplit; ++s) {
    ak += *(const f32x4*)(ws + (size_t)s * 2 * (size_t)slab + e);
    av += *(const f32x4*)(ws + (size_t)s * 2 * (size_t)slab + slab + e);
  }
  *(u32x2*)(dk + e) = (u32x2){pack_bf16x2(ak[0], ak[1]), pack_bf16x2(ak[2], ak[3])};
  *(u32x2*)(dv + e) = (u32x2){pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3])};
}

// Varlen form of the reduce: workgroup (sequence, key/value head, 128-row block) adds up the
// rows of that sequence only, so tokens that no sequence covers stay unwritten in dK and dV
// (and their workspace rows, which no split wrote, are never read).
__global__ __launch_bounds__(256) void fa2_bwd_kv_reduce_varlen_kernel(BwdParams p) {
  const int rb = blockIdx.x, bk = blockIdx.y;
  const int bi = bk / p.Hkv, hk = bk - bi * p.Hkv;
  int tok0, len;
  seq_range<true>(p, bi, tok0, len);
  const int r0 = rb * 128;
  if (r0 >= len) return;
  const int rows = min(128, len - r0);
  const int c4 = p.dg / 4;                    // float4 groups per row
  const size_t base = (kv_plane<true>(p, bi, hk) + (size_t)tok0 + (size_t)r0) * (size_t)p.dg;
  for (int t = threadIdx.x; t < rows * c4; t += 256) {
    const size_t e = base + (size_t)(t / c4) * (size_t)p.dg + (size_t)(t % c4) * 4;
    f32x4 ak = *(const f32x4*)(p.kv_ws + e);
    f32x4 av = *(const f32x4*)(p.kv_ws + p.ws_slab + e);
    for (int s = 1; s < p.hsplit; ++s) {
      ak += *(const f32x4*)(p.kv_ws + (size_t)s * 2 * (size_t)p.ws_slab + e);
      av += *(const f32x4*)(p.kv_ws + (size_t)s * 2 * (size_t)p.ws_slab + p.ws_slab + e);
    }
    *(u32x2*)(p.dk + e) = (u32x2){pack_bf16x2(ak[0], ak[1]), pack_bf16x2(ak[2], ak[3])};
    *(u32x2*)(p.dv + e) = (u32x2){pack_bf16x2(av[0], av[1]), pack_bf16x2(av[2], av[3])};
  }
}

// ---- host side ------------------------------------------------------------------------

typedef const void* KernelFn;

struct BwdKernels {
  int dq_bc;
  int dq_br;
  int dq_threads;
  int dkdv_threads;
  int dkdv_bk;           // keys per dK/dV workgroup
  int dkdv_occ;          // dK/dV waves per SIMD
  KernelFn dq[2][2];     // [varlen][causal]
  KernelFn dkdv[2][2];
  // Persistent forms, taken by varlen calls outside graph capture: workgroups per CU (0: none)
  // and the kernels, [causal].
  int dq_wg_per_cu = 0;
  int dkdv_wg_per_cu = 0;
  KernelFn dq_persist[2] = {nullptr, nullptr};
  KernelFn dkdv_persist[2] = {nullptr, nullptr};
};

template <int D, int BC_DQ, int NW_DQ, int OCC_DQ, int NW_DKDV, int OCC_DKDV, int BQ_DKDV, bool KLDS,
          int LA_DQ, int LA_DKDV, int LA_DKDV_ACC, bool PERSIST_DQ, bool PERSIST_DKDV>
BwdKernels make_bwd() {
  BwdKernels k;
  k.dq_bc = BC_DQ;
  k.dq_br = DqTile<D, BC_DQ, NW_DQ>::BR;
  k.dq_threads = DqTile<D, BC_DQ, NW_DQ>::THREADS;
  k.dkdv_threads = DkvTile<D, BQ_DKDV, NW_DKDV>::THREADS;
  k.dkdv_bk = DkvTile<D, BQ_DKDV, NW_DKDV>::BK;
  k.dkdv_occ = OCC_DKDV;
  k.dq[0][0] = (KernelFn)&fa2_bwd_dq_kernel<D, BC_DQ, false, false, NW_DQ, OCC_DQ, LA_DQ>;
  k.dq[0][1] = (KernelFn)&fa2_bwd_dq_kernel<D, BC_DQ, true, false, NW_DQ, OCC_DQ, LA_DQ>;
  k.dq[1][0] = (KernelFn)&fa2_bwd_dq_kernel<D, BC_DQ, false, true, NW_DQ, OCC_DQ, LA_DQ>;
  k.dq[1][1] = (KernelFn)&fa2_bwd_dq_kernel<D, BC_DQ, true, true, NW_DQ, OCC_DQ, LA_DQ>;
  k.dkdv[0][0] = (KernelFn)&fa2_bwd_dkdv_kernel<D, BQ_DKDV, false, false, NW_DKDV, OCC_DKDV, KLDS, LA_DKDV, LA_DKDV_ACC>;
  k.dkdv[0][1] = (KernelFn)&fa2_bwd_dkdv_kernel<D, BQ_DKDV, true, false, NW_DKDV, OCC_DKDV, KLDS, LA_DKDV, LA_DKDV_ACC>;
  k.dkdv[1][0] = (KernelFn)&fa2_bwd_dkdv_kernel<D, BQ_DKDV, false, true, NW_DKDV, OCC_DKDV, KLDS, LA_DKDV, LA_DKDV_ACC>;
  k.dkdv[1][1] = (KernelFn)&fa2_bwd_dkdv_kernel<D, BQ_DKDV, true, true, NW_DKDV, OCC_DKDV, KLDS, LA_DKDV, LA_DKDV_ACC>;
  if constexpr (PERSIST_DQ) {
    k.dq_wg_per_cu = 4 * OCC_DQ / NW_DQ;
    k.dq_persist[0] = (KernelFn)&fa2_bwd_dq_kernel_persist<D, BC_DQ, false, true, NW_DQ, OCC_DQ, LA_DQ>;
    k.dq_persist[1] = (KernelFn)&fa2_bwd_dq_kernel_persist<D, BC_DQ, true, true, NW_DQ, OCC_DQ, LA_DQ>;
  }
  if constexpr (PERSIST_DKDV) {
    k.dkdv_wg_per_cu = 4 * OCC_DKDV / NW_DKDV;
    k.dkdv_persist[0] =
        (KernelFn)&fa2_bwd_dkdv_kernel_persist<D, BQ_DKDV, false, true, NW_DKDV, OCC_DKDV, KLDS, LA_DKDV, LA_DKDV_ACC>;
    k.dkdv_persist[1] =
        (KernelFn)&fa2_bwd_dkdv_kernel_persist<D, BQ_DKDV, true, true, NW_DKDV, OCC_DKDV, KLDS, LA_DKDV, LA_DKDV_ACC>;
  }
  return k;
}

const BwdKernels* bwd_kernels(int d) {
  // <D, dQ key tile, dQ waves, dQ waves per SIMD, dK/dV waves, dK/dV waves per SIMD, dK/dV
  //  query step, K rows of dK/dV in LDS, look-aheads of the dQ S/dP chain, the dK/dV S/dP
  //  chain and the dK/dV accumulation, persistent dQ and dK/dV forms for varlen calls>:
  //  chosen so each kernel keeps as many waves per SIMD as its registers allow (d = 128
  //  dK/dV: 32-query steps and K in LDS bring it from one to two), then the deepest
  //  look-ahead that still fits without spills and measured fastest. The persistent forms
  //  pay at d = 128 and 256 (16 packed sequences: +8% and +20%); at d = 64, with three and
  //  four workgroups per CU, the dQ form measured 4% slower and the dK/dV form no faster.
  static const BwdKernels k64 = make_bwd<64, 32, 4, 4, 4, 3, 32, true, 1, 2, 0, false, false>();
  static const BwdKernels k128 = make_bwd<128, 32, 4, 2, 4, 2, 32, true, 4, 2, 0, true, true>();
  // d = 256: the dQ^T, dK^T and dV^T accumulators are 128 registers each, so both kernels run
  // one wave per SIMD (dK/dV: 129 KB of LDS, one workgroup per CU).
  static const BwdKernels k256 = make_bwd<256, 32, 4, 1, 4, 1, 32, true, 4, 4, 2, true, true>();
  return d == 64 ? &k64 : d == 128 ? &k128 : d == 256 ? &k256 : nullptr;
}

bool aligned_to(const void* ptr, uintptr_t a) { return ((uintptr_t)ptr & (a - 1)) == 0; }

// Query-head splits of the dK/dV kernel in a fixed-length call with grouped- or multi-query
// heads. Unsplit, the kernel has one wave per 32 keys of each key/value head, which leaves
// SIMDs idle when there are few key/value heads (B=1, H_kv=2, N=16384: 1024 waves, where two
// per SIMD of the 256 CUs take 2048). Causal key blocks carry unequal work (the first sees
// every query, the last one tile), so there the kernel needs about four waves per slot for
// the heaviest-first order to even them out; with one per slot the heaviest block sets the
// time (measured: two splits, one wave per slot, 615 TFLOP/s against 837 without groups).
// Returns the smallest divisor S of g that gives at least occ waves per SIMD (four times
// that when causal), else g; 1 when g == 1.
constexpr long long kBwdSimds = 1024;   // 256 CUs x 4 SIMDs
int bwd_head_split(long long B, int H_kv, int g, int N, int occ, bool causal) {
  const long long waves = B * H_kv * (((long long)N + 31) / 32);
  const long long target = kBwdSimds * occ * (causal ? 4 : 1);
  for (int S = 1; S < g; ++S)
    if (g % S == 0 && waves * S >= target) return S;
  return g;
}

// Head dimensions of the backward: multiples of 8 up to 256, run on the D = 64, 128 or 256
// kernels with padded columns as in the forward. Q, O, dO, K and V padded columns are either zero in
// registers (rows loaded by lanes) or duplicates of real columns of the same row (tiles staged
// to LDS); every product that reaches a written output pairs a padded column with a zero one,
// and gradient columns past d are never written.
bool bwd_head_dim(int d) { return d >= 8 && d <= 256 && d % 8 == 0; }
int bwd_padded_dim(int d) { return d <= 64 ? 64 : d <= 128 ? 128 : 256; }

// One launch of a backward kernel over num_wg work items: one workgroup per item, or, for the
// persistent form (wg_per_cu > 0), min(num_wg, CUs * wg_per_cu) workgroups sharing a work
// queue whose counters come from the library's pool.
int bwd_kernel_launch(KernelFn plain, KernelFn persist, int wg_per_cu, int threads, BwdParams& p,
                      long long num_wg, int dev, void* stream) {
  if (persist && wg_per_cu > 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      return FA2_ERR_NO_DEVICE;
    unsigned int* ctr = nullptr;
    const int st = fa2_internal::queue_counters(dev, &ctr);
    if (st != FA2_OK) return st;
    int total = (int)num_wg;
    const long long grid = num_wg < (long long)cus * wg_per_cu ? num_wg : (long long)cus * wg_per_cu;
    void* args[] = {&p, &ctr, &total};
    return hipLaunchKernel(persist, dim3((unsigned)grid), dim3((unsigned)threads), args, 0,
                           (hipStream_t)stream) == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
  }
  void* args[] = {&p};
  return hipLaunchKernel(plain, dim3((unsigned)num_wg), dim3((unsigned)threads), args, 0,
                         (hipStream_t)stream) == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}

int bwd_launch(const BwdKernels& kk, bool varlen, bool causal, BwdParams p, int nblk_q, int nblk_k,
               long long npairs_q, long long npairs_k, void* stream) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return FA2_ERR_NO_DEVICE;
  const int v = varlen ? 1 : 0, c = causal ? 1 : 0;
  // Varlen calls take the persistent forms where they exist: the blocks past the end of the
  // shorter sequences cost a queue fetch instead of a workgroup launch. Under stream capture a graph would keep
  // the counter sets it captured, so captured calls take the one-block-per-workgroup kernels
  // (same blocks, same results).
  bool persist = varlen;
  if (persist) {
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing((hipStream_t)stream, &cap) != hipSuccess) return FA2_ERR_LAUNCH;
    persist = cap == hipStreamCaptureStatusNone;
  }
  p.nblk = nblk_q;
  // Per-XCD pair ranges for fixed-length batches; varlen uses the plain heaviest-first order
  // (with unequal sequence lengths the per-XCD ranges get unequal shares, as in the forward).
  p.heads_per_xcd = (!varlen && npairs_q % 8 == 0) ? (int)(npairs_q / 8) : 0;
  int st = bwd_kernel_launch(kk.dq[v][c], persist ? kk.dq_persist[c] : nullptr, kk.dq_wg_per_cu,
                             kk.dq_threads, p, nblk_q * npairs_q, dev, stream);
  if (st != FA2_OK) return st;
  BwdParams p2 = p;
  p2.nblk = nblk_k;
  const long long items_k = npairs_k * p.hsplit;   // (pair, split) work items per key block
  p2.heads_per_xcd = (!varlen && items_k % 8 == 0) ? (int)(items_k / 8) : 0;
  st = bwd_kernel_launch(kk.dkdv[v][c], persist ? kk.dkdv_persist[c] : nullptr, kk.dkdv_wg_per_cu,
                         kk.dkdv_threads, p2, nblk_k * items_k, dev, stream);
  if (st != FA2_OK || p.hsplit == 1) return st;
  if (varlen) {
    hipLaunchKernelGGL(fa2_bwd_kv_reduce_varlen_kernel, dim3((unsigned)((p.N + 127) / 128), (unsigned)npairs_k),
                       dim3(256), 0, (hipStream_t)stream, p);
  } else {
    const long long nthr = p.ws_slab / 4;
    hipLaunchKernelGGL(fa2_bwd_kv_reduce_kernel, dim3((unsigned)((nthr + 255) / 256)), dim3(256), 0,
                       (hipStream_t)stream, (const float*)p.kv_ws, p.ws_slab, p.hsplit, p.dk, p.dv);
  }
  return hipGetLastError() == hipSuccess ? FA2_OK : FA2_ERR_LAUNCH;
}

int bwd_check(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dout, const void* dq, const void* dk, const void* dv, const float* delta,
              int d, float scale) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !delta) return FA2_ERR_NULL_PTR;
  if (!bwd_head_dim(d)) return FA2_ERR_UNSUPPORTED_HEADDIM;
  const void* b16[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* ptr : b16)
    if (!aligned_to(ptr, 16)) return FA2_ERR_MISALIGNED;
  if (!aligned_to(lse, 4) || !aligned_to(delta, 4)) return FA2_ERR_MISALIGNED;
  if (!isfinite(scale)) return FA2_ERR_BAD_SCALE;
  return FA2_OK;
}

void bwd_fill(BwdParams& p, const void* q, const void* k, const void* v, const void* o,
              const float* lse, const void* dout, void* dq, void* dk, void* dv, float* delta,
              float scale) {
  p.q = (const uint16_t*)q;
  p.k = (const uint16_t*)k;
  p.v = (const uint16_t*)v;
  p.o = (const uint16_t*)o;
  p.lse = lse;
  p.dout = (const uint16_t*)dout;
  p.dq = (uint16_t*)dq;
  p.dk = (uint16_t*)dk;
  p.dv = (uint16_t*)dv;
  p.delta = delta;
  p.hsplit = 1;
  p.kv_ws = nullptr;
  p.ws_slab = 0;
  p.c = fmaxf(fabsf(scale) * kLog2e, 1e-30f);
  p.scale = scale;
  p.qflip = scale < 0.f ? 0x80008000u : 0u;
}

// Fixed-length backward; split allows query-head splits of the dK/dV kernel (fa2_bwd_ws).
int bwd_fixed(const void* q, const void* k, const void* v, const void* o, const float* lse,
              const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H, int H_kv,
              int N, int d, int causal, float scale, bool split, void* workspace,
              long long workspace_bytes, void* stream) {
  if (B <= 0 || H <= 0 || H_kv <= 0 || H % H_kv != 0 || N < 0) return FA2_ERR_BAD_SHAPE;
  if (N == 0) return bwd_head_dim(d) ? FA2_OK : FA2_ERR_UNSUPPORTED_HEADDIM;
  int st = bwd_check(q, k, v, o, lse, dout, dq, dk, dv, delta, d, scale);
  if (st != FA2_OK) return st;
  const long long nblk = ((long long)N + 127) / 128;   // most blocks any kernel launches
  const long long pq = (long long)B * H, pk = (long long)B * H_kv;
  if (nblk * pq > 0x7fffffffLL || pq * (long long)N > 0x7fffffffLL) return FA2_ERR_TOO_LARGE;
  const BwdKernels& kk = *bwd_kernels(bwd_padded_dim(d));
  const int S = split ? bwd_head_split(B, H_kv, H / H_kv, N, kk.dkdv_occ, causal != 0) : 1;
  const long long slab = pk * (long long)N * d;         // elements of dK (or dV)
  if (S > 1) {
    if (!workspace) return FA2_ERR_NULL_PTR;
    if (!aligned_to(workspace, 16)) return FA2_ERR_MISALIGNED;
    if (workspace_bytes < (long long)S * 2 * slab * (long long)sizeof(float)) return FA2_ERR_SCRATCH_TOO_SMALL;
  }
  BwdParams p;
  bwd_fill(p, q, k, v, o, lse, dout, dq, dk, dv, delta, scale);
  p.cu_seqlens = nullptr;
  p.nb = B;
  p.dg = d;
  p.H = H;
  p.Hkv = H_kv;
  p.g = H / H_kv;
  p.N = N;
  p.T = N;
  p.hsplit = S;
  p.kv_ws = S > 1 ? (float*)workspace : nullptr;
  p.ws_slab = S > 1 ? slab : 0;
  const long long nblk_q = ((long long)N + kk.dq_br - 1) / kk.dq_br;
  const long long nblk_k = ((long long)N + kk.dkdv_bk - 1) / kk.dkdv_bk;
  if (nblk_k * pk * S > 0x7fffffffLL) return FA2_ERR_TOO_LARGE;
  return bwd_launch(kk, false, causal != 0, p, (int)nblk_q, (int)nblk_k, pq, pk, stream);
}

// Varlen backward; split allows query-head splits of the dK/dV kernel (fa2_bwd_varlen_ws).
int bwd_varlen_impl(const void* q, const void* k, const void* v, const void* o, const float* lse,
                    const void* dout, void* dq, void* dk, void* dv, float* delta,
                    const int* cu_seqlens, int num_seqs, int max_seqlen, int total_tokens, int H,
                    int H_kv, int d, int causal, float scale, bool split, void* workspace,
                    long long workspace_bytes, void* stream) {
  if (H <= 0 || H_kv <= 0 || H % H_kv != 0 || num_seqs < 0 || max_seqlen < 0 || total_tokens < 0)
    return FA2_ERR_BAD_SHAPE;
  if (num_seqs == 0 || total_tokens == 0 || max_seqlen == 0)
    return bwd_head_dim(d) ? FA2_OK : FA2_ERR_UNSUPPORTED_HEADDIM;
  if (!cu_seqlens) return FA2_ERR_NULL_PTR;
  if (!aligned_to(cu_seqlens, 4)) return FA2_ERR_MISALIGNED;
  int st = bwd_check(q, k, v, o, lse, dout, dq, dk, dv, delta, d, scale);
  if (st != FA2_OK) return st;
  const long long nblk = ((long long)max_seqlen + 127) / 128;   // most blocks any kernel launches
  const long long pq = (long long)num_seqs * H, pk = (long long)num_seqs * H_kv;
  if (nblk * pq > 0x7fffffffLL || (long long)H * total_tokens > 0x7fffffffLL) return FA2_ERR_TOO_LARGE;
  BwdParams p;
  bwd_fill(p, q, k, v, o, lse, dout, dq, dk, dv, delta, scale);
  p.cu_seqlens = cu_seqlens;
  p.nb = num_seqs;
  p.dg = d;
  p.H = H;
  p.Hkv = H_kv;
  p.g = H / H_kv;
  p.N = max_seqlen;
  p.T = total_tokens;
  const BwdKernels& kk = *bwd_kernels(bwd_padded_dim(d));
  const int S = split ? bwd_head_split(1, H_kv, H / H_kv, total_tokens, kk.dkdv_occ, causal != 0) : 1;
  const long long slab = (long long)H_kv * total_tokens * d;
  if (S > 1) {
    if (!workspace) return FA2_ERR_NULL_PTR;
    if (!aligned_to(workspace, 16)) return FA2_ERR_MISALIGNED;
    if (workspace_bytes < (long long)S * 2 * slab * (long long)sizeof(float)) return FA2_ERR_SCRATCH_TOO_SMALL;
  }
  p.hsplit = S;
  p.kv_ws = S > 1 ? (float*)workspace : nullptr;
  p.ws_slab = S > 1 ? slab : 0;
  const long long nblk_q = ((long long)max_seqlen + kk.dq_br - 1) / kk.dq_br;
  const long long nblk_k = ((long long)max_seqlen + kk.dkdv_bk - 1) / kk.dkdv_bk;
  if (nblk_k * pk * S > 0x7fffffffLL) return FA2_ERR_TOO_LARGE;
  return bwd_launch(kk, true, causal != 0, p, (int)nblk_q, (int)nblk_k, pq, pk, stream);
}


}  // namespace

extern "C" {

long long fa2_bwd_workspace_bytes(int B, int H, int H_kv, int N, int d, int causal) {
  if (B <= 0 || H <= 0 || H_kv <= 0 || H % H_kv != 0 || N <= 0 || !bwd_head_dim(d)) return 0;
  const BwdKernels& kk = *bwd_kernels(bwd_padded_dim(d));
  const int S = bwd_head_split(B, H_kv, H / H_kv, N, kk.dkdv_occ, causal != 0);
  return S > 1 ? (long long)S * 2 * B * H_kv * (long long)N * d * (long long)sizeof(float) : 0;
}

int fa2_bwd(const void* q, const void* k, const void* v, const void* o, const float* lse,
            const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H, int H_kv,
            int N, int d, int causal, float scale, void* stream) {
  return bwd_fixed(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, H_kv, N, d, causal, scale, false,
                   nullptr, 0, stream);
}

int fa2_bwd_ws(const void* q, const void* k, const void* v, const void* o, const float* lse,
               const void* dout, void* dq, void* dk, void* dv, float* delta, int B, int H, int H_kv,
               int N, int d, int causal, float scale, void* workspace, long long workspace_bytes,
               void* stream) {
  return bwd_fixed(q, k, v, o, lse, dout, dq, dk, dv, delta, B, H, H_kv, N, d, causal, scale, true,
                   workspace, workspace_bytes, stream);
}

int fa2_bwd_varlen(const void* q, const void* k, const void* v, const void* o, const float* lse,
                   const void* dout, void* dq, void* dk, void* dv, float* delta,
                   const int* cu_seqlens, int num_seqs, int max_seqlen, int total_tokens, int H,
                   int H_kv, int d, int causal, float scale, void* stream) {
  return bwd_varlen_impl(q, k, v, o, lse, dout, dq, dk, dv, delta, cu_seqlens, num_seqs, max_seqlen,
                         total_tokens, H, H_kv, d, causal, scale, false, nullptr, 0, stream);
}

long long fa2_bwd_varlen_workspace_bytes(int num_seqs, int max_seqlen, int total_tokens, int H, int H_kv,
                                         int d, int causal) {
  if (num_seqs <= 0 || max_seqlen <= 0 || total_tokens <= 0 || H <= 0 || H_kv <= 0 || H % H_kv != 0 ||
      !bwd_head_dim(d))
    return 0;
  const BwdKernels& kk = *bwd_kernels(bwd_padded_dim(d));
  // T keys per key/value head stand in for the sequences' keys (equal when cu covers all tokens).
  const int S = bwd_head_split(1, H_kv, H / H_kv, total_tokens, kk.dkdv_occ, causal != 0);
  return S > 1 ? (long long)S * 2 * H_kv * (long long)total_tokens * d * (long long)sizeof(float) : 0;
}

int fa2_bwd_varlen_ws(const void* q, const void* k, const void* v, const void* o, const float* lse,
                      const void* dout, void* dq, void* dk, void* dv, float* delta,
                      const int* cu_seqlens, int num_seqs, int max_seqlen, int total_tokens, int H,
                      int H_kv, int d, int causal, float scale, void* workspace, long long workspace_bytes,
                      void* stream) {
  return bwd_varlen_impl(q, k, v, o, lse, dout, dq, dk, dv, delta, cu_seqlens, num_seqs, max_seqlen,
                         total_tokens, H, H_kv, d, causal, scale, true, workspace, workspace_bytes, stream);
}

}  // extern "C"
