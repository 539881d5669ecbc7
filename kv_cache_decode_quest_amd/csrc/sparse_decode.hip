// sparse_decode.hip -- attention over the selected pages (the explicit-KV
// attention view of the SparseEngine digest, Method key points), as a split-K
// paged flash-decode followed by a log-sum-exp merge.
//
// Work split.  A work-group owns one (request, KV head) row and one split of
// that row's selected pages; its waves take the split's pages round-robin.
// All G q heads of the KV head are processed together, so each K/V page is
// read from HBM once per step.  Each wave keeps, per head, a running max m,
// a running sum l and an fp32 accumulator acc[D] (online softmax, logits in
// base 2: x = sm_scale * log2(e) * q.k); the waves of a work-group merge
// through LDS and write one partial (acc, m, l) per head; merge_kernel then
// combines the splits.
//
// bf16 path (matrix cores).  A wave takes a round of PPW pages at a time:
// it issues the K loads of all of them, then the V loads, and folds the
// whole round into its running softmax with one max / sum update:
//   S   = K q^T    C[16 tokens][16 heads] += K[16 tokens][32 d] * q^T[32 d][16 heads]
//                  (v_mfma_f32_16x16x32_bf16, D/32 steps per 16-token tile; K
//                  pages are token-major, so each lane loads 16 contiguous bytes)
//   O^T += V^T P^T C[16 d][16 heads] += V^T[16 d][16 tokens] * P^T[16 tokens][16 heads]
//                  (v_mfma_f32_16x16x16_bf16, one step per 16-token tile and
//                  16-channel tile; V pages are dim-major, so each lane loads 4
//                  consecutive tokens of one channel as 8 contiguous bytes)
// The first product leaves lane l with head l % 16 and tokens 4*(l/16)..+3,
// which is exactly the lane's B operand of the second: softmax weights never
// leave their registers.  The second product's result keeps the head in the
// lane's column too, so a lane's running max, running sum and accumulator
// all belong to one head and rescaling is lane-local.  For the second
// product each fp32 weight is split into two bf16 values hi + lo (lo = the
// rounding error of hi), and both go through the matrix cores, so the weights
// keep about 16 significant bits instead of bf16's 8.  Heads past G are zero
// columns of q^T.
#include <algorithm>

#include "quest_device.h"
#include "quest_launch.h"
#include "topk_select.h"

namespace quest {

constexpr float kLog2e = 1.4426950408889634f;

// XCDs of an MI355X.  With a grid of a multiple of kXcds work-groups,
// work-group b runs on XCD b mod kXcds; xcd_item numbers the work items so
// that consecutive items share an XCD (item = XCD x stride + b/kXcds, stride
// = grid/kXcds), or keeps item = b when stride is 0.  The stride is a kernel
// argument rather than gridDim, so the item is known after the one scalar
// load of the arguments (0.3 us per step at batch 8 x 128000 against a
// branch that read the grid size on its own).
constexpr unsigned kXcds = 8;
__device__ __forceinline__ int xcd_item(unsigned b, int stride) {
  return stride ? (int)((b % kXcds) * (unsigned)stride + b / kXcds) : (int)b;
}
// Whether a decode grid of `blocks` work-groups (n_split per row) and its
// merge grid of `mblocks` can be numbered XCD-major with every row's splits
// and merge on one XCD.  Used by the fused kernel only, whose grid is one
// wave of work-groups (0.3 us per step at batch 8 x 128000); the standalone
// decode's multi-wave grids ran slower numbered this way (the dense
// reference 509 against 389 us), so they keep the plain order.
static bool xcd_placement(unsigned blocks, int n_split, unsigned mblocks) {
  return n_split > 1 && blocks % kXcds == 0 && (blocks / kXcds) % (unsigned)n_split == 0 &&
         mblocks % kXcds == 0;
}

// Pages folded into the running softmax per update.  The loads of a round
// are issued group by group (K then V of each group), so a group's update
// can start while later groups are still in flight.
constexpr int kPagesPerUpdate = 2;

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// A pair of fp32 weights as packed bf16 hi = RNE(p) and lo = RNE(p - hi),
// each pair converted by one v_cvt_pk_bf16_f32 (round to nearest even).
__device__ __forceinline__ void split_bf16x2(float p0, float p1, uint32_t &hi, uint32_t &lo) {
  const bf16x2 h = {(__bf16)p0, (__bf16)p1};
  hi = __builtin_bit_cast(uint32_t, h);
  const float r0 = p0 - __uint_as_float(hi << 16);
  const float r1 = p1 - __uint_as_float(hi & 0xffff0000u);
  const bf16x2 lw = {(__bf16)r0, (__bf16)r1};
  lo = __builtin_bit_cast(uint32_t, lw);
}

// ---------------------------------------------------------------------------
// bf16 matrix-core kernel
// ---------------------------------------------------------------------------
template <int D, int P>
struct PageRegs {
  static constexpr int TT = P / 16;     // 16-token tiles
  static constexpr int KC = D / 32;     // 32-channel chunks of q.k
  static constexpr int NT = D / 16;     // 16-channel tiles of the output
  uint4 k[TT][KC];
  uint2 v[TT][NT];
};

// Which token a row of a 16-token tile holds.  Pages of 32 and 64 tokens are
// attended in pairs of tiles (32 tokens): in a pair's first tile, matrix row i
// holds the pair's token 8*(i/4) + i%4, in its second tile token
// 8*(i/4) + 4 + i%4.  The four logits lane (col, grp) then gets from each
// tile of the pair (rows 4*grp .. +3) are the pair's tokens 8*grp .. 8*grp + 7
// in order: the 8 consecutive tokens of one channel that the lane loads as 16
// contiguous bytes of the dim-major V page, and the K slots of one
// v_mfma_f32_16x16x32_bf16 of O^T += V^T P^T.  Pages of 16 tokens (one tile)
// keep row i = token i.
template <int TT>
__device__ __forceinline__ int k_row_token(int tt, int row) {
  return TT >= 2 ? 32 * (tt >> 1) + 8 * (row >> 2) + 4 * (tt & 1) + (row & 3) : tt * 16 + row;
}
// The first of the four tokens lane slot group `tok0` = 4*grp holds in tile tt
// (the logits of S and the V values of the same lane both follow it).
template <int TT>
__device__ __forceinline__ int lane_token0(int tt, int tok0) {
  return TT >= 2 ? 32 * (tt >> 1) + 2 * tok0 + 4 * (tt & 1) : tt * 16 + tok0;
}

// K (token-major): lane (col, grp) takes the token of row col of tile tt,
// channels c*32 + 8*grp .. +7 -- its A operand of S = K q^T.
template <int D, int P>
__device__ __forceinline__ void load_k(PageRegs<D, P> &pr, const uint16_t *__restrict__ kp,
                                       int col, int grp) {
  constexpr int TT = PageRegs<D, P>::TT;
#pragma unroll
  for (int tt = 0; tt < TT; ++tt)
#pragma unroll
    for (int c = 0; c < PageRegs<D, P>::KC; ++c)
      pr.k[tt][c] = *(const uint4 *)(kp + k_row_token<TT>(tt, col) * D + c * 32 + grp * 8);
}

// V (dim-major): lane (col, grp) takes channel nt*16 + col: one tile, tokens
// 4*grp .. +3 (8 bytes); a pair of tiles, the pair's tokens 8*grp .. +7 (16
// bytes, the first four for the pair's first tile) -- its A operand of
// O^T = V^T P^T.
template <int D, int P>
__device__ __forceinline__ void load_v(PageRegs<D, P> &pr, const uint16_t *__restrict__ vp,
                                       int col, int grp) {
  constexpr int TT = PageRegs<D, P>::TT;
  if constexpr (TT >= 2) {
#pragma unroll
    for (int pp = 0; pp < TT / 2; ++pp)
#pragma unroll
      for (int nt = 0; nt < PageRegs<D, P>::NT; ++nt) {
        const uint4 w = *(const uint4 *)(vp + (nt * 16 + col) * P + pp * 32 + grp * 8);
        pr.v[2 * pp][nt] = make_uint2(w.x, w.y);
        pr.v[2 * pp + 1][nt] = make_uint2(w.z, w.w);
      }
  } else {
#pragma unroll
    for (int nt = 0; nt < PageRegs<D, P>::NT; ++nt)
      pr.v[0][nt] = *(const uint2 *)(vp + (nt * 16 + col) * P + grp * 4);
  }
}

// 8-token pages: a 16-token tile holds page a in tokens 0..7 and page b in
// tokens 8..15.  K rows: lane (col, grp) takes token col of the tile; V: lane
// (col, grp) takes tokens 4*grp .. +3, i.e. slots 4*(grp & 1) .. +3 of page a
// (grp < 2) or b.
template <int D>
__device__ __forceinline__ void load_k_half(PageRegs<D, 16> &pr, const uint16_t *__restrict__ kpa,
                                            const uint16_t *__restrict__ kpb, int col, int grp) {
  const uint16_t *kp = (col < 8 ? kpa : kpb) + (col & 7) * D;
#pragma unroll
  for (int c = 0; c < PageRegs<D, 16>::KC; ++c)
    pr.k[0][c] = *(const uint4 *)(kp + c * 32 + grp * 8);
}

template <int D>
__device__ __forceinline__ void load_v_half(PageRegs<D, 16> &pr, const uint16_t *__restrict__ vpa,
                                            const uint16_t *__restrict__ vpb, int col, int grp) {
  const uint16_t *vp = (grp < 2 ? vpa : vpb) + (grp & 1) * 4;
#pragma unroll
  for (int nt = 0; nt < PageRegs<D, 16>::NT; ++nt)
    pr.v[0][nt] = *(const uint2 *)(vp + (nt * 16 + col) * 8);
}

// One round of the online softmax over the NPG pages a wave holds, for all
// heads of the group at once: the logits of every page on the matrix cores,
// one running-max / running-sum update for the whole round, then
// O^T += V^T P^T on the matrix cores.  Lane (col, grp) owns head `col`: its
// running max m and sum l, and accumulator channels nt*16 + 4*grp .. +3, so
// the rescale needs no cross-lane traffic.  valid[u] is the number of tokens
// of page u that take part (0 for an unused slot).
//
// kPack (groups of at most 8 heads): columns 8..15 of the products carry no
// head, so lane (col >= 8) takes over the logits of head col - 8 (one DPP
// row shift) and feeds that head's lo weights to the second product while
// lane col - 8 feeds the hi weights: one matrix-core step per tile instead of
// two, and accumulator columns h and h + 8 add up to head h.
//
// Validity: token lane_token0(tt, tok0) + e of the lane takes part iff it is
// below lim[u]; full[u] (uniform) says every token of tile-page u does.
// Pages of two or more tiles multiply P.V a pair of tiles (32 tokens) at a
// time on v_mfma_f32_16x16x32_bf16 (see k_row_token).
template <int D, int P, int NPG, bool kPack>
__device__ __forceinline__ void attend_round(PageRegs<D, P> *pg, const int *lim,
                                             const bool *full, int tok0, const bf16x8 *qop,
                                             float scale2, int col, float &m, float &l,
                                             f32x4 *acc) {
  using PR = PageRegs<D, P>;
  constexpr float kNegInf = -__builtin_huge_valf();
  // logits: lane holds head `col` (kPack: head col mod 8), tokens tt*16 + 4*grp + e
  f32x4 s[NPG][PR::TT];
  float pmax = kNegInf;
#pragma unroll
  for (int u = 0; u < NPG; ++u) {
#pragma unroll
    for (int tt = 0; tt < PR::TT; ++tt) {
      f32x4 c4 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < PR::KC; ++c)
        c4 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, pg[u].k[tt][c]),
                                                     qop[c], c4, 0, 0, 0);
      if constexpr (kPack) {
        // lanes 8..15 of each row take lanes 0..7's values; lanes 0..7 have
        // no source 8 lanes below inside the row and keep their own
#pragma unroll
        for (int e = 0; e < 4; ++e)
          c4[e] = __uint_as_float(dpp_row<kRowShr8>(__float_as_uint(c4[e]), __float_as_uint(c4[e])));
      }
      if (full[u]) {                        // a full page (uniform branch)
#pragma unroll
        for (int e = 0; e < 4; ++e) s[u][tt][e] = c4[e] * scale2;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e)
          s[u][tt][e] = lane_token0<PR::TT>(tt, tok0) + e < lim[u] ? c4[e] * scale2 : kNegInf;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) pmax = fmaxf(pmax, s[u][tt][e]);
    }
  }
  pmax = max_over_rows(pmax);
  const float m_new = fmaxf(m, pmax);
  // while no token has been seen m stays -inf: subtract 0 then, so every
  // weight is exp2(-inf) = 0 rather than NaN
  const float m_sub = (m_new == kNegInf) ? 0.f : m_new;
  const float alpha = (m == kNegInf) ? 0.f : exp2_fast(m - m_new);
  // weights as a sum of two bf16 values (hi + lo), so the matrix-core
  // product keeps about 16 significant bits of every weight
  float psum = 0.f;
  s16x4 phi[NPG][PR::TT], plo[NPG][PR::TT];
#pragma unroll
  for (int u = 0; u < NPG; ++u) {
#pragma unroll
    for (int tt = 0; tt < PR::TT; ++tt) {
      float p[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = exp2_fast(s[u][tt][e] - m_sub);
        psum += p[e];
      }
      uint32_t h01, l01, h23, l23;
      split_bf16x2(p[0], p[1], h01, l01);
      split_bf16x2(p[2], p[3], h23, l23);
      phi[u][tt] = __builtin_bit_cast(s16x4, make_uint2(h01, h23));
      plo[u][tt] = __builtin_bit_cast(s16x4, make_uint2(l01, l23));
    }
  }
  psum = sum_over_rows(psum);
  l = l * alpha + psum;
  m = m_new;
#pragma unroll
  for (int nt = 0; nt < PR::NT; ++nt)
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[nt][e] *= alpha;
#pragma unroll
  for (int u = 0; u < NPG; ++u) {
    // The slots of a partial page past its valid tokens may hold anything
    // (NaN included): zero their V values, since a zero weight times NaN is
    // still NaN.
    if (!full[u]) {
#pragma unroll
      for (int tt = 0; tt < PR::TT; ++tt) {
        const int t0 = lane_token0<PR::TT>(tt, tok0);
        const uint32_t mx = (t0 + 0 < lim[u] ? 0x0000ffffu : 0u) |
                            (t0 + 1 < lim[u] ? 0xffff0000u : 0u);
        const uint32_t my = (t0 + 2 < lim[u] ? 0x0000ffffu : 0u) |
                            (t0 + 3 < lim[u] ? 0xffff0000u : 0u);
#pragma unroll
        for (int nt = 0; nt < PR::NT; ++nt) {
          pg[u].v[tt][nt].x &= mx;
          pg[u].v[tt][nt].y &= my;
        }
      }
    }
    if constexpr (PR::TT >= 2) {
      // a pair of tiles per product: K slots 8*grp + j are the pair's tokens
      // 8*grp + j for both operands (tile 2pp gives j < 4, tile 2pp+1 j >= 4)
      auto pair = [](s16x4 a, s16x4 b) {
        return __builtin_bit_cast(bf16x8, make_uint4(__builtin_bit_cast(uint2, a).x,
                                                     __builtin_bit_cast(uint2, a).y,
                                                     __builtin_bit_cast(uint2, b).x,
                                                     __builtin_bit_cast(uint2, b).y));
      };
#pragma unroll
      for (int pp = 0; pp < PR::TT / 2; ++pp) {
        const bf16x8 whi = pair(phi[u][2 * pp], phi[u][2 * pp + 1]);
        const bf16x8 wlo = pair(plo[u][2 * pp], plo[u][2 * pp + 1]);
#pragma unroll
        for (int nt = 0; nt < PR::NT; ++nt) {
          const uint2 v0 = pg[u].v[2 * pp][nt], v1 = pg[u].v[2 * pp + 1][nt];
          const bf16x8 vv = __builtin_bit_cast(bf16x8, make_uint4(v0.x, v0.y, v1.x, v1.y));
          if constexpr (kPack) {
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, col < 8 ? whi : wlo, acc[nt],
                                                              0, 0, 0);
          } else {
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, whi, acc[nt], 0, 0, 0);
            acc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv, wlo, acc[nt], 0, 0, 0);
          }
        }
      }
    } else {
#pragma unroll
      for (int nt = 0; nt < PR::NT; ++nt) {
        const s16x4 vv = __builtin_bit_cast(s16x4, pg[u].v[0][nt]);
        if constexpr (kPack) {
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vv, col < 8 ? phi[u][0] : plo[u][0],
                                                              acc[nt], 0, 0, 0);
        } else {
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vv, phi[u][0], acc[nt], 0, 0, 0);
          acc[nt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vv, plo[u][0], acc[nt], 0, 0, 0);
        }
      }
    }
  }
}

// One split of one selection row on a work-group of kWaves waves (8, or 16
// with half the pages per wave: the same pages per round).  ids(i) is the
// row's i-th selected page (read for some i past the split or the count,
// whose value is then ignored); count() the row's selected count, at most
// max_k; ctx_of(r) request r's length.  Writes the split's partial (acc, m,
// l) per head, or, with final_out (a row of one split), the row's output
// acc / l in bf16 directly — what the merge would compute from that single
// partial, bit for bit.  kAhead (splits of several rounds): the next round's
// page ids and page-table entries are looked up right after the current
// round's K/V loads are issued, so each later round starts its K/V loads at
// once; results are the same bit for bit.
template <int D, int P, bool kPack, int kWaves, bool kAhead, bool kNonEmpty = false,
          typename Ids, typename Count, typename CtxOf>
__device__ __forceinline__ void decode_split(
    int row, int split, int R, int G, int Hkv, int gdiv, int64_t pool, int max_pages,
    int max_k, int n_split, int pps, float scale2, const uint16_t *__restrict__ q,
    const uint16_t *__restrict__ k_cache, const uint16_t *__restrict__ v_cache,
    const int32_t *__restrict__ page_table, CtxOf ctx_of, Ids ids, Count count,
    float *__restrict__ partial, uint16_t *__restrict__ final_out = nullptr) {
  static_assert(kWaves == kDecodeWaves || kWaves == 2 * kDecodeWaves, "wave count");
  // 8-token pages are attended two to a 16-token tile ("tile page")
  constexpr bool kHalf = P < 16;
  constexpr int TP = kHalf ? 16 : P;
  constexpr int SUB = kHalf ? 2 : 1;    // pages per tile page
  using PR = PageRegs<D, TP>;
  constexpr int PPW = pages_per_wave(P, D) * kDecodeWaves / kWaves;
  static_assert(PPW >= SUB, "at least one tile page per wave");
  constexpr int NV = PPW / SUB;         // tile pages per wave and round
  constexpr int kLdsRow = D + 4;       // padded so the 16-byte stores below spread over banks
  __shared__ float lds_m[kWaves][16];
  __shared__ float lds_l[kWaves][16];
  __shared__ __align__(16) float lds_acc[kWaves][16][kLdsRow];

  const int lane = threadIdx.x & 63;
  // wave index as a scalar: the page lookups below become scalar loads
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  // selection row `row` = request r, row hr of the request: q heads
  // hr*G .. hr*G+G-1 of the request, reading KV head hr / gdiv
  const int r = row / R, hr = row - r * R, g = hr / gdiv;
  const int first = split * pps;
  const int32_t *pt = page_table + (int64_t)r * max_pages;
  const int64_t page_elems = (int64_t)P * D;
  // The first round of page ids is read together with the row's count and
  // length (ids past the count are ignored below), so the chain to the first
  // K/V load is ids -> page table -> K/V.
  constexpr int kRound = kWaves * PPW;
  int sel0[PPW];
#pragma unroll
  for (int u = 0; u < PPW; ++u) {
    const int i = first + wave * PPW + u;
    sel0[u] = ids(i < max_k ? i : max_k - 1);
  }
  const int jfirst = ids(first < max_k ? first : max_k - 1);
  const int nsel = count();
  const int ctx = ctx_of(r);
  // (kNonEmpty: the caller only passes splits that hold pages, so the count
  // is not waited for here and its load goes out with the page ids'; 0.45 us
  // per step on the ragged batch, one scalar round trip per split)
  if (!kNonEmpty && first >= nsel) {               // no page in this split:
    if (final_out) {                                // a row with no page outputs zeros
      for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x)
        Elem<uint16_t>::store(final_out, (int64_t)row * G * D + idx, 0.f);
      return;
    }
    float *mine = partial + ((int64_t)row * n_split + split) * G * (D + 2);
    for (int h = threadIdx.x; h < G; h += blockDim.x) {   // an empty partial
      mine[h * (D + 2) + D] = -__builtin_huge_valf();
      mine[h * (D + 2) + D + 1] = 0.f;
    }
    return;
  }
  const int last = min(nsel, first + pps);
  const int n = pages_in(ctx, P, max_pages);

  // q^T operand: column `col` = head, K slots of group `grp` (zero past G).
  // Loads here and below are unconditional, from clamped in-bounds
  // addresses: a load under a branch makes the compiler drain every
  // outstanding load at the join.
  bf16x8 qop[PR::KC];
  {
    const uint16_t *qh = q + ((int64_t)r * R * G + (int64_t)hr * G + (col < G ? col : 0)) * D;
    uint4 w[PR::KC];
#pragma unroll
    for (int c = 0; c < PR::KC; ++c) w[c] = *(const uint4 *)(qh + c * 32 + grp * 8);
#pragma unroll
    for (int c = 0; c < PR::KC; ++c)
      qop[c] = __builtin_bit_cast(bf16x8, col < G ? w[c] : make_uint4(0, 0, 0, 0));
  }

  f32x4 acc[PR::NT];
#pragma unroll
  for (int nt = 0; nt < PR::NT; ++nt) acc[nt] = (f32x4){0.f, 0.f, 0.f, 0.f};
  float m = -__builtin_huge_valf();     // running max of head `col` (base-2 logits)
  float l = 0.f;                        // running sum of head `col`

  // The physical page and valid-token count of selected position i with
  // logical id j (slots past the split, or with an id outside the request,
  // re-read the split's first page, a cache hit, with no valid token).
  auto lookup = [&](int i, int j, int64_t &ph_out, int &valid_out) {
    const bool live = i < last && j >= 0 && j < n;
    const int jj = live ? j : ((jfirst >= 0 && jfirst < n) ? jfirst : 0);
    const int64_t ph = pt[jj];
    const bool ok = ph >= 0 && ph < pool;
    ph_out = ok ? ph : 0;
    valid_out = (live && ok) ? min(P, ctx - j * P) : 0;
  };
  int64_t next_phys[PPW];
  int next_valid[PPW];
  // Each round, wave w takes PPW consecutive selected pages.
  for (int base = first; base < last; base += kRound) {
    const int p0 = base + wave * PPW;
    int64_t phys[PPW];
    int valid[PPW];
    if (!kAhead || base == first) {
#pragma unroll
      for (int u = 0; u < PPW; ++u) {
        const int i = p0 + u;
        lookup(i, (base == first) ? sel0[u] : ids(i < last ? i : last - 1), phys[u], valid[u]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < PPW; ++u) {
        phys[u] = next_phys[u];
        valid[u] = next_valid[u];
      }
    }
    // per update group: all K, then all V (the logits need only the K loads)
    constexpr int UPG = kPagesPerUpdate < NV ? kPagesPerUpdate : NV;
    PR pg[NV];
    auto kbase = [&](int u) { return k_cache + (phys[u] * Hkv + g) * page_elems; };
    auto vbase = [&](int u) { return v_cache + (phys[u] * Hkv + g) * page_elems; };
#pragma unroll
    for (int g0 = 0; g0 < NV; g0 += UPG) {
#pragma unroll
      for (int v = g0; v < g0 + UPG; ++v) {
        if constexpr (kHalf) load_k_half<D>(pg[v], kbase(2 * v), kbase(2 * v + 1), col, grp);
        else load_k<D, TP>(pg[v], kbase(v), col, grp);
      }
#pragma unroll
      for (int v = g0; v < g0 + UPG; ++v) {
        if constexpr (kHalf) load_v_half<D>(pg[v], vbase(2 * v), vbase(2 * v + 1), col, grp);
        else load_v<D, TP>(pg[v], vbase(v), col, grp);
      }
    }
    // keep every load of the round ahead of the first wait on any of them
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (kAhead) {
      // the next round's lookups (unconditional, clamped; unused after the
      // last round), in flight while this round's pages arrive
#pragma unroll
      for (int u = 0; u < PPW; ++u) {
        const int i = p0 + kRound + u;
        lookup(i, ids(i < last ? i : last - 1), next_phys[u], next_valid[u]);
      }
    }
    // validity per tile page: this lane's tokens 4*grp .. +3 lie in page
    // 2v + (grp >> 1) of a half tile, as slots 4*(grp & 1) .. +3
    int lim[NV];
    bool full[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
      if constexpr (kHalf) {
        lim[v] = grp < 2 ? valid[2 * v] : valid[2 * v + 1];
        full[v] = valid[2 * v] >= P && valid[2 * v + 1] >= P;
      } else {
        lim[v] = valid[v];
        full[v] = valid[v] >= P;
      }
    }
    const int tok0 = kHalf ? 4 * (grp & 1) : 4 * grp;
#pragma unroll
    for (int g0 = 0; g0 < NV; g0 += UPG)
      attend_round<D, TP, UPG, kPack>(pg + g0, lim + g0, full + g0, tok0, qop, scale2, col, m,
                                      l, acc);
  }

  // merge the waves of this work-group
  if (grp == 0) {
    lds_m[wave][col] = m;
    lds_l[wave][col] = l;
  }
#pragma unroll
  for (int nt = 0; nt < PR::NT; ++nt)
    *(f32x4 *)&lds_acc[wave][col][nt * 16 + 4 * grp] = acc[nt];
  __syncthreads();
  float *out = partial + ((int64_t)row * n_split + split) * G * (D + 2);
  for (int idx = threadIdx.x; idx < G * D; idx += blockDim.x) {
    const int h = idx / D, d = idx - h * D;
    float M = -__builtin_huge_valf();
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, lds_m[w][h]);
    float a = 0.f, L = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mw = lds_m[w][h];
      const float f = (mw == -__builtin_huge_valf()) ? 0.f : exp2_fast(mw - M);
      const float aw = kPack ? lds_acc[w][h][d] + lds_acc[w][h + 8][d] : lds_acc[w][h][d];
      a += f * aw;
      L += f * lds_l[w][h];
    }
    if (final_out) {
      Elem<uint16_t>::store(final_out, ((int64_t)row * G + h) * D + d, L > 0.f ? a / L : 0.f);
      continue;
    }
    float *ph = out + h * (D + 2);
    ph[d] = a;
    if (d == 0) {
      ph[D] = M;
      ph[D + 1] = L;
    }
  }
}

template <int D, int P, bool kPack, bool kAhead>
__global__ __launch_bounds__(kDecodeWaves * 64) void sparse_decode_mfma_kernel(
    int R, int G, int Hkv, int gdiv, int64_t pool, int max_pages, int max_k, int n_split,
    int pps, float scale2, const uint16_t *__restrict__ q, const uint16_t *__restrict__ k_cache,
    const uint16_t *__restrict__ v_cache, const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ ctx_lens, const int32_t *__restrict__ sel_pages,
    const int32_t *__restrict__ num_sel, float *__restrict__ partial) {
  const int split = blockIdx.x % n_split;
  const int row = blockIdx.x / n_split;
  const int32_t *sel = sel_pages + (int64_t)row * max_k;
  decode_split<D, P, kPack, kDecodeWaves, kAhead>(
      row, split, R, G, Hkv, gdiv, pool, max_pages, max_k, n_split, pps, scale2, q, k_cache,
      v_cache, page_table, [&](int r) { return ctx_lens[r]; }, [&](int i) { return sel[i]; },
      [&] { return min(num_sel[row], max_k); }, partial);
}

// The live-split form of the bf16 decode: the grid (kLiveGrid work-groups)
// takes only the splits that hold selected pages.  Every work-group counts
// each row's live splits from the selection counts, scans them into LDS
// (units_end[x] = live splits of rows 0..x), and attends live splits b, b +
// A, b + 2 A, ... mapped back to (row, split) by a binary search over the
// scan.  Dead splits are never visited and write no partial; the merge reads
// only the live ones.  A ragged batch, whose grid in the per-(row, split)
// form is sized by its longest row, then spreads the real work evenly.
// A is the number of work-groups that take part: with U live splits and a
// grid of N, every one of A = ceil(U / ceil(U / N)) work-groups attends
// ceil(U / N) splits (the last one fewer) and the others exit.  The splits
// stream at the HBM rate while every work-group has one in flight, so equal
// shares keep the chip busy to the end; with all N taking part, the last
// round of splits would run on a fraction of the CUs (U = 1376, N = 256:
// 96 work-groups for the last 11 us of a 78 us launch).  kAhead: splits of
// several rounds look each next round's pages up ahead, as in decode_split.
template <int D, int P, bool kPack, bool kAhead>
__global__ __launch_bounds__(kDecodeWaves * 64) void sparse_decode_live_kernel(
    int rows, int R, int G, int Hkv, int gdiv, int64_t pool, int max_pages, int max_k,
    int n_split, int pps, float scale2, const uint16_t *__restrict__ q,
    const uint16_t *__restrict__ k_cache, const uint16_t *__restrict__ v_cache,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ ctx_lens,
    const int32_t *__restrict__ sel_pages, const int32_t *__restrict__ num_sel,
    float *__restrict__ partial) {
  __shared__ uint32_t units_end[kLiveRows];
  __shared__ uint32_t wave_total[kDecodeWaves];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  auto units_of = [&](int count) -> uint32_t {
    const int k = min(count, max_k);
    return k > 0 ? (uint32_t)((k + pps - 1) / pps) : 0u;
  };
  // inclusive scan of the rows' live splits: thread t owns rows 2t and 2t+1
  // (both counts read at once from indices clamped into the rows, then
  // masked: loads under the row test were drained one after the other)
  static_assert(2 * kDecodeWaves * 64 >= kLiveRows, "two rows per thread");
  const int x0 = 2 * threadIdx.x;
  const int c0 = num_sel[min(x0, rows - 1)];
  const int c1 = num_sel[min(x0 + 1, rows - 1)];
  const uint32_t u0 = x0 < rows ? units_of(c0) : 0u;
  const uint32_t u1 = x0 + 1 < rows ? units_of(c1) : 0u;
  const uint32_t incl = wave_incl_sum(u0 + u1);
  if (lane == 63) wave_total[wave] = incl;
  __syncthreads();
  uint32_t before = 0;
#pragma unroll
  for (int w = 0; w < kDecodeWaves; ++w) before += w < wave ? wave_total[w] : 0u;
  if (x0 < rows) units_end[x0] = before + incl - u1;
  if (x0 + 1 < rows) units_end[x0 + 1] = before + incl;
  __syncthreads();
  const uint32_t total = units_end[rows - 1];
  const uint32_t per = (total + gridDim.x - 1) / gridDim.x;
  const uint32_t active = per > 0 ? (total + per - 1) / per : 0u;
  for (uint32_t u = blockIdx.x; u < total && blockIdx.x < active; u += active) {
    // the row holding live split u: the first x with units_end[x] > u
    int lo = 0, hi = rows - 1;
    while (lo < hi) {
      const int mid = (lo + hi) >> 1;
      if (units_end[mid] > u) hi = mid;
      else lo = mid + 1;
    }
    const int row = lo;
    const int split = (int)(u - (row > 0 ? units_end[row - 1] : 0u));
    // the previous split's work-group merge has finished reading its LDS
    if (u != blockIdx.x) __syncthreads();
    // a live split is one of the row's first ceil(count / pps), so its first
    // position is below the count: decode_split skips its empty-split test
    const int32_t *sel = sel_pages + (int64_t)row * max_k;
    decode_split<D, P, kPack, kDecodeWaves, kAhead, true>(
        row, split, R, G, Hkv, gdiv, pool, max_pages, max_k, n_split, pps, scale2, q, k_cache,
        v_cache, page_table, [&](int r) { return ctx_lens[r]; }, [&](int i) { return sel[i]; },
        [&] { return min(num_sel[row], max_k); }, partial);
  }
}

// ---------------------------------------------------------------------------
// Fused top-k + decode (bf16).  Every work-group of a row runs the row's
// selection itself (1024 threads, the row's scores read from global memory),
// keeps the page ids of its own split in LDS, then attends them with 16
// waves of half the pages each (the same pages per round as the 8-wave
// kernel, so the partials have the same form).  Each split also writes the
// positions of the row's selection it attends, split 0 the count and the
// unused tail.  The selection is repeated by every split of a
// row: it pays where the grid fits in one wave of resident work-groups (one
// per CU at this kernel's LDS size), so the repeats run side by side instead
// of one launch before the decode.  The plan (fused_plan) splits a row only
// as far as that allows; a row of one split (many rows) writes its output
// directly, and then no merge runs at all.
// ---------------------------------------------------------------------------
constexpr int kFusedWaves = 2 * kDecodeWaves;
static_assert(kFusedWaves * kWave == kTopkThreads, "the fused kernel runs the 1024-thread selection");
template <int D, int P, bool kPack, bool kAhead>
__global__ __launch_bounds__(kTopkThreads) void topk_decode_mfma_kernel(
    int R, int G, int Hkv, int gdiv, int64_t pool, int max_pages, int max_k, int n_split,
    int pps, int n_sink, int n_recent, float scale2, const uint16_t *__restrict__ q,
    const uint16_t *__restrict__ k_cache, const uint16_t *__restrict__ v_cache,
    const int32_t *__restrict__ page_table, const int32_t *__restrict__ ctx_lens,
    const float *__restrict__ scores, const int32_t *__restrict__ budget_tokens,
    int32_t *__restrict__ sel_pages, int32_t *__restrict__ num_sel,
    float *__restrict__ partial, uint16_t *__restrict__ out_final, int xcd_stride) {
  __shared__ TopkShared sh;
  __shared__ int32_t split_pages[kMaxFusedPages];
  const int tid = threadIdx.x, lane = lane_id(), wave = tid >> 6;
  const int lin = xcd_item(blockIdx.x, xcd_stride);
  const int split = lin % n_split;
  const int row = lin / n_split;
  const int r = row / R;
  const int log2p = __builtin_ctz(P);                 // the page size is a power of two
  const float *s = scores + (int64_t)row * max_pages;
  const int span = reg_span(max_pages);               // pages per wave of a register row
  float sv[kPerThread];                               // the row fits in registers
#pragma unroll
  for (int i = 0; i < kPerThread; ++i) {
    const int j = wave * span + i * kWave + lane;
    sv[i] = s[min(j, max_pages - 1)];
  }
  const int ctx = ctx_lens[r];
  int n, k;
  row_size(ctx, budget_tokens[r], log2p, max_pages, max_k, n, k);
  const int first = split * pps;
  int32_t *out = sel_pages + (int64_t)row * max_k;
  if (split == 0) {
    if (tid == 0) num_sel[row] = k;
    for (int i = k + tid; i < max_k; i += kTopkThreads) out[i] = -1;
  }
  // positions of the split at or past the row's count k are never emitted
  // (and never live below): they hold 0; the emitted ones are disjoint
  for (int i = tid; i < pps; i += kTopkThreads)
    if (first + i >= k) split_pages[i] = 0;
  // each split writes the positions it attends (the splits' ranges tile
  // [0, k)), so no work-group carries the whole row's stores into the wait
  // its decode starts with (the compiler drains the stores there: 0.4-0.6 us
  // off the kernel at batch 8 x 128000)
  auto emit = [&](int pos, int j) {
    const unsigned x = (unsigned)(pos - first);
    if (x < (unsigned)pps) {
      split_pages[x] = j;
      out[pos] = j;
    }
  };
  if (n_sink > 0 || n_recent > 0) select_row<true, true>(sh, s, sv, span, n, k, n_sink, n_recent, emit);
  else select_row<true, false>(sh, s, sv, span, n, k, 0, 0, emit);
  __syncthreads();
  // any index is clamped into the list
  decode_split<D, P, kPack, kFusedWaves, kAhead>(
      row, split, R, G, Hkv, gdiv, pool, max_pages, max_k, n_split, pps, scale2, q, k_cache,
      v_cache, page_table, [&](int) { return ctx; },
      [&](int i) {
        const int x = i - first;
        return split_pages[x < 0 ? 0 : (x < pps ? x : pps - 1)];
      },
      [&] { return k; }, partial, n_split == 1 ? out_final : nullptr);
}

// ---------------------------------------------------------------------------
// fp32 kernel (vector ALUs): one work-group walks its split's pages in order,
// staging each K and V page in LDS.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void sparse_decode_valu_kernel(
    int R, int G, int Hkv, int gdiv, int D, int P, int64_t pool, int max_pages, int max_k,
    int n_split, int pps, float scale2, const float *__restrict__ q,
    const float *__restrict__ k_cache,
    const float *__restrict__ v_cache, const int32_t *__restrict__ page_table,
    const int32_t *__restrict__ ctx_lens, const int32_t *__restrict__ sel_pages,
    const int32_t *__restrict__ num_sel, float *__restrict__ partial) {
  extern __shared__ float lds[];
  float *q_s = lds;                 // [G][D]
  float *k_s = q_s + G * D;         // [P][D]
  float *v_s = k_s + P * D;         // [D][P]
  float *p_s = v_s + P * D;         // [G][P]
  float *m_s = p_s + G * P;         // [G]
  float *l_s = m_s + G;             // [G]
  float *a_s = l_s + G;             // [G] rescale factors

  const int split = blockIdx.x % n_split;
  const int row = blockIdx.x / n_split;
  const int r = row / R, hr = row - r * R, g = hr / gdiv;
  const int nsel = min(num_sel[row], max_k);
  const int first = split * pps;
  if (first >= nsel) {                             // no page in this split:
    float *mine = partial + ((int64_t)row * n_split + split) * G * (D + 2);
    for (int h = threadIdx.x; h < G; h += blockDim.x) {   // an empty partial
      mine[h * (D + 2) + D] = -__builtin_huge_valf();
      mine[h * (D + 2) + D + 1] = 0.f;
    }
    return;
  }
  const int last = min(nsel, first + pps);
  const int ctx = ctx_lens[r];
  const int n = pages_in(ctx, P, max_pages);
  const int32_t *sel = sel_pages + (int64_t)row * max_k;
  const int32_t *pt = page_table + (int64_t)r * max_pages;

  const float *qg = q + ((int64_t)r * R * G + (int64_t)hr * G) * D;
  for (int x = threadIdx.x; x < G * D; x += blockDim.x) q_s[x] = qg[x];
  for (int h = threadIdx.x; h < G; h += blockDim.x) {
    m_s[h] = -__builtin_huge_valf();
    l_s[h] = 0.f;
  }
  float acc[8];                      // pairs (h, d) = threadIdx.x + 256 * e
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  __syncthreads();

  for (int i = first; i < last; ++i) {
    const int j = sel[i];
    if (j < 0 || j >= n) continue;
    const int64_t phys = pt[j];
    if (phys < 0 || phys >= pool) continue;
    const int valid = min(P, ctx - j * P);
    const float *kp = k_cache + (phys * Hkv + g) * (int64_t)P * D;
    const float *vp = v_cache + (phys * Hkv + g) * (int64_t)P * D;
    for (int x = threadIdx.x; x < P * D; x += blockDim.x) {
      k_s[x] = kp[x];
      v_s[x] = vp[x];
    }
    __syncthreads();
    for (int x = threadIdx.x; x < G * P; x += blockDim.x) {
      const int h = x / P, t = x - h * P;
      float dot = 0.f;
      for (int d = 0; d < D; ++d) dot += q_s[h * D + d] * k_s[t * D + d];
      p_s[x] = t < valid ? dot * scale2 : -__builtin_huge_valf();
    }
    __syncthreads();
    for (int h = threadIdx.x; h < G; h += blockDim.x) {
      float pm = -__builtin_huge_valf();
      for (int t = 0; t < P; ++t) pm = fmaxf(pm, p_s[h * P + t]);
      const float m_old = m_s[h];
      const float m_new = fmaxf(m_old, pm);
      const float alpha = (m_old == -__builtin_huge_valf()) ? 0.f : exp2_fast(m_old - m_new);
      float sum = 0.f;
      for (int t = 0; t < P; ++t) {
        const float w = exp2_fast(p_s[h * P + t] - m_new);
        p_s[h * P + t] = w;
        sum += w;
      }
      l_s[h] = l_s[h] * alpha + sum;
      m_s[h] = m_new;
      a_s[h] = alpha;
    }
    __syncthreads();
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int x = threadIdx.x + 256 * e;
      if (x < G * D) {
        const int h = x / D, d = x - h * D;
        float a = acc[e] * a_s[h];
        for (int t = 0; t < valid; ++t) a += p_s[h * P + t] * v_s[d * P + t];
        acc[e] = a;
      }
    }
    __syncthreads();
  }
  float *base = partial + ((int64_t)row * n_split + split) * G * (D + 2);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int x = threadIdx.x + 256 * e;
    if (x < G * D) {
      const int h = x / D, d = x - h * D;
      base[h * (D + 2) + d] = acc[e];
      if (d == 0) {
        base[h * (D + 2) + D] = m_s[h];
        base[h * (D + 2) + D + 1] = l_s[h];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// merge: out[r][h] = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s
// One work-group per (request, q head), one thread per channel.  Splits are
// taken kChunk at a time with all of their loads issued together (the max
// and sum are the same address across the work-group), merged online.  A
// bf16 row has at most 8 splits once the batch has 32 selection rows or
// more, so its merge is one round trip to memory; a batch of fewer rows
// gives each row up to ceil(256 / rows) splits, 32 per round trip.  kChunk
// is the fewest of 8, 16 and 32 that holds the row's splits: the slots of a
// chunk past n_split re-load the chunk's first split and the wave still
// waits for them (a chunk of 32 for 8 splits cost 1.3 us per step at batch
// 8 x 128000 and 2.8 us on the ragged batch).
// ---------------------------------------------------------------------------
constexpr int kMergeChunk = 32;

// A row's partials are its first ceil(count / pps) splits (the live ones;
// the per-(row, split) kernels also write empty partials, max -inf and sum
// 0, past them, while the live-split kernel writes nothing there).  The
// partials are loaded for all n_split splits at once, without waiting for
// the count, and the splits past the live ones are masked.
template <typename T, int kChunk>
__global__ __launch_bounds__(128) void merge_kernel(int R, int G, int D, int n_split, int pps,
                                                    int max_k, const int32_t *__restrict__ num_sel,
                                                    const float *__restrict__ partial,
                                                    T *__restrict__ out, int xcd_stride) {
  // r * Hq + h
  const int hq = xcd_item(blockIdx.x, xcd_stride);
  const int Hq = R * G;
  const int r = hq / Hq, h = hq - r * Hq;
  const int g = h / G, hl = h - g * G;
  const int row = r * R + g;
  const int64_t stride = (int64_t)G * (D + 2);
  // every argument the loads and the merge need is in registers before the
  // row's count is requested: a later argument load would make the compiler
  // wait for all outstanding scalar loads, the count's included, before the
  // partials' loads go out
  asm volatile("" ::"s"(partial), "s"(out), "s"(num_sel), "s"(max_k), "s"(pps), "s"(n_split));
  const int count = num_sel[row];
  // A zero the compiler cannot see through, added to the base address: the
  // statistics loads below then stay vector loads into vector registers (as
  // uniform loads, 32 splits' statistics and addresses overflow the scalar
  // registers).
  int lane0;
  asm volatile("v_mov_b32 %0, 0" : "=v"(lane0));
  const float *base =
      partial + (int64_t)row * n_split * stride + (int64_t)hl * (D + 2) + lane0;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float M = -__builtin_huge_valf(), L = 0.f, a = 0.f;
    for (int s0 = 0; s0 < n_split; s0 += kChunk) {
      float mv[kChunk], lv[kChunk], av[kChunk];
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const float *p = base + (s0 + u < n_split ? s0 + u : s0) * stride;
        mv[u] = p[D];
        lv[u] = p[D + 1];
        av[u] = p[d];
      }
      // the chunk's loads are out before the count is waited for (the opaque
      // copy keeps the count's first use here: the compiler would otherwise
      // hoist it above the loop, and the wait with it; 0.5 us per step at
      // batch 8 x 128000)
      __builtin_amdgcn_sched_barrier(0);
      int c = count;
      asm volatile("" : "+v"(c));
      const int cnt = min(c, max_k);
      const int live = cnt > 0 ? min(n_split, (cnt + pps - 1) / pps) : 0;
      float cm = M;
#pragma unroll
      for (int u = 0; u < kChunk; ++u)
        if (s0 + u < live) cm = fmaxf(cm, mv[u]);
      if (cm == -__builtin_huge_valf()) continue;  // nothing but empty splits so far
      const float f0 = (M == -__builtin_huge_valf()) ? 0.f : exp2_fast(M - cm);
      a *= f0;
      L *= f0;
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        // an empty split (max -inf) leaves its accumulator unwritten: select,
        // never multiply it by a zero weight
        if (s0 + u < live && mv[u] != -__builtin_huge_valf()) {
          const float f = exp2_fast(mv[u] - cm);
          a += f * av[u];
          L += f * lv[u];
        }
      }
      M = cm;
    }
    Elem<T>::store(out, (int64_t)hq * D + d, L > 0.f ? a / L : 0.f);
  }
}

static hipError_t launch_merge(const Dims &dm, int batch, const DecodePlan &plan, int max_k,
                               const int32_t *num_sel, const float *workspace, void *out,
                               hipStream_t stream, int xcd_stride = 0) {
  const unsigned mblocks = (unsigned)((long)batch * dm.Hq);
  // splits per round trip: the fewest of 8, 16, 32 that hold the row's
  // splits (slots past n_split would re-load the first one)
#define QUEST_MERGE(TT, CH)                                                               \
  hipLaunchKernelGGL((merge_kernel<TT, CH>), dim3(mblocks), dim3(128), 0, stream, dm.R,    \
                     dm.Gcols, dm.D, plan.n_split, plan.pages_per_split, max_k, num_sel,  \
                     workspace, (TT *)out, xcd_stride)
#define QUEST_MERGE_T(TT)                                                                 \
  do {                                                                                    \
    if (plan.n_split <= 8) QUEST_MERGE(TT, 8);                                            \
    else if (plan.n_split <= 16) QUEST_MERGE(TT, 16);                                     \
    else QUEST_MERGE(TT, kMergeChunk);                                                    \
  } while (0)
  if (dm.dtype == 1) QUEST_MERGE_T(uint16_t);
  else QUEST_MERGE_T(float);
#undef QUEST_MERGE_T
#undef QUEST_MERGE
  return hipGetLastError();
}

hipError_t launch_decode(const Dims &dm, int batch, const void *q,
                         const void *k_cache, const void *v_cache,
                         const int32_t *page_table, const int32_t *ctx_lens,
                         const int32_t *sel_pages, const int32_t *num_sel,
                         int max_k, float sm_scale, void *out,
                         float *workspace, hipStream_t stream) {
  const DecodePlan plan = decode_plan(dm, batch, max_k);
  const float scale2 = sm_scale * kLog2e;
  const unsigned blocks = (unsigned)decode_grid(dm, batch, max_k);
  const bool live = decode_live(dm, batch);
  const int rows = batch * dm.R;
  // splits of several rounds look the next round's pages up ahead
  const bool ahead =
      dm.dtype == 1 && plan.pages_per_split > kDecodeWaves * pages_per_wave(dm.P, dm.D);
  if (dm.dtype == 1) {
#define QUEST_DECODE(DD, PP)                                                              \
  do {                                                                                    \
    if (dm.Gcols <= 8) QUEST_DECODE_G(DD, PP, true);                                      \
    else QUEST_DECODE_G(DD, PP, false);                                                   \
  } while (0)
#define QUEST_DECODE_G(DD, PP, PK)                                                        \
  do {                                                                                    \
    if (live && ahead)                                                                    \
      hipLaunchKernelGGL((sparse_decode_live_kernel<DD, PP, PK, true>), dim3(blocks),     \
                         dim3(kDecodeWaves * 64), 0, stream, rows, dm.R, dm.Gcols, dm.Hkv, \
                         dm.gdiv, dm.pool, dm.max_pages, max_k, plan.n_split,             \
                         plan.pages_per_split, scale2, (const uint16_t *)q,               \
                         (const uint16_t *)k_cache, (const uint16_t *)v_cache,            \
                         page_table, ctx_lens, sel_pages, num_sel, workspace);            \
    else if (live)                                                                        \
      hipLaunchKernelGGL((sparse_decode_live_kernel<DD, PP, PK, false>), dim3(blocks),    \
                         dim3(kDecodeWaves * 64), 0, stream, rows, dm.R, dm.Gcols, dm.Hkv, \
                         dm.gdiv, dm.pool, dm.max_pages, max_k, plan.n_split,             \
                         plan.pages_per_split, scale2, (const uint16_t *)q,               \
                         (const uint16_t *)k_cache, (const uint16_t *)v_cache,            \
                         page_table, ctx_lens, sel_pages, num_sel, workspace);            \
    else if (ahead)                                                                       \
      hipLaunchKernelGGL((sparse_decode_mfma_kernel<DD, PP, PK, true>), dim3(blocks),     \
                         dim3(kDecodeWaves * 64), 0, stream, dm.R, dm.Gcols, dm.Hkv,      \
                         dm.gdiv, dm.pool, dm.max_pages, max_k, plan.n_split,             \
                         plan.pages_per_split, scale2, (const uint16_t *)q,               \
                         (const uint16_t *)k_cache, (const uint16_t *)v_cache,            \
                         page_table, ctx_lens, sel_pages, num_sel, workspace);            \
    else                                                                                  \
      hipLaunchKernelGGL((sparse_decode_mfma_kernel<DD, PP, PK, false>), dim3(blocks),    \
                         dim3(kDecodeWaves * 64), 0, stream, dm.R, dm.Gcols, dm.Hkv,      \
                         dm.gdiv, dm.pool, dm.max_pages, max_k, plan.n_split,             \
                         plan.pages_per_split, scale2, (const uint16_t *)q,               \
                         (const uint16_t *)k_cache, (const uint16_t *)v_cache,            \
                         page_table, ctx_lens, sel_pages, num_sel, workspace);            \
  } while (0)
    if (dm.D == 128 && dm.P == 16) QUEST_DECODE(128, 16);
    else if (dm.D == 128 && dm.P == 32) QUEST_DECODE(128, 32);
    else if (dm.D == 128 && dm.P == 64) QUEST_DECODE(128, 64);
    else if (dm.D == 128 && dm.P == 8) QUEST_DECODE(128, 8);
    else if (dm.D == 64 && dm.P == 8) QUEST_DECODE(64, 8);
    else if (dm.D == 64 && dm.P == 16) QUEST_DECODE(64, 16);
    else if (dm.D == 64 && dm.P == 32) QUEST_DECODE(64, 32);
    else QUEST_DECODE(64, 64);
#undef QUEST_DECODE
#undef QUEST_DECODE_G
  } else {
    const size_t lds = sizeof(float) * ((size_t)dm.Gcols * dm.D + 2 * (size_t)dm.P * dm.D +
                                        (size_t)dm.Gcols * dm.P + 3 * (size_t)dm.Gcols);
    hipLaunchKernelGGL(sparse_decode_valu_kernel, dim3(blocks), dim3(256), lds, stream,
                       dm.R, dm.Gcols, dm.Hkv, dm.gdiv, dm.D, dm.P, dm.pool, dm.max_pages,
                       max_k, plan.n_split,
                       plan.pages_per_split, scale2, (const float *)q, (const float *)k_cache,
                       (const float *)v_cache, page_table, ctx_lens, sel_pages, num_sel,
                       workspace);
  }
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;
  return launch_merge(dm, batch, plan, max_k, num_sel, workspace, out, stream);
}

hipError_t launch_topk_decode(const Dims &dm, int batch, const void *q, const void *k_cache,
                              const void *v_cache, const int32_t *page_table,
                              const int32_t *ctx_lens, const float *scores,
                              const int32_t *budget_tokens, int max_k, int n_sink,
                              int n_recent, float sm_scale, int32_t *sel_pages,
                              int32_t *num_sel, void *out, float *workspace,
                              hipStream_t stream) {
  if (!topk_decode_fused(dm, batch, max_k)) {
    const hipError_t err = launch_topk(dm, batch, scores, ctx_lens, budget_tokens, max_k,
                                       n_sink, n_recent, sel_pages, num_sel, stream);
    if (err != hipSuccess) return err;
    return launch_decode(dm, batch, q, k_cache, v_cache, page_table, ctx_lens, sel_pages,
                         num_sel, max_k, sm_scale, out, workspace, stream);
  }
  const DecodePlan plan = fused_plan(dm, batch, max_k);
  const float scale2 = sm_scale * kLog2e;
  const unsigned blocks = (unsigned)((long)batch * dm.R * plan.n_split);
  const unsigned mblocks = (unsigned)((long)batch * dm.Hq);
  // XCD placement (a performance choice only; results do not depend on where
  // a work-group runs): the dispatcher deals work-groups to the 8 XCDs in
  // turn, so work-group b runs on XCD b mod 8.  Numbering the work items
  // XCD-major keeps the splits of a row, and the merge of its heads, on one
  // XCD, where the score row and the partials stay in that XCD's L2.
  const bool xcd = xcd_placement(blocks, plan.n_split, mblocks);
  // splits of several rounds look the next round's pages up ahead (a round:
  // 16 waves of half the 8-wave kernel's pages)
  const bool ahead = plan.pages_per_split > kDecodeWaves * pages_per_wave(dm.P, dm.D);
#define QUEST_FUSED(DD, PP)                                                               \
  do {                                                                                    \
    if (dm.Gcols <= 8) QUEST_FUSED_G(DD, PP, true);                                       \
    else QUEST_FUSED_G(DD, PP, false);                                                    \
  } while (0)
#define QUEST_FUSED_G(DD, PP, PK)                                                         \
  do {                                                                                    \
    if (ahead) QUEST_FUSED_A(DD, PP, PK, true);                                           \
    else QUEST_FUSED_A(DD, PP, PK, false);                                                \
  } while (0)
#define QUEST_FUSED_A(DD, PP, PK, AH)                                                     \
  hipLaunchKernelGGL((topk_decode_mfma_kernel<DD, PP, PK, AH>), dim3(blocks),             \
                     dim3(kTopkThreads), 0, stream, dm.R, dm.Gcols, dm.Hkv, dm.gdiv,      \
                     dm.pool, dm.max_pages, max_k, plan.n_split, plan.pages_per_split,    \
                     n_sink, n_recent, scale2, (const uint16_t *)q,                       \
                     (const uint16_t *)k_cache, (const uint16_t *)v_cache, page_table,    \
                     ctx_lens, scores, budget_tokens, sel_pages, num_sel, workspace,      \
                     (uint16_t *)out, xcd ? (int)(blocks / kXcds) : 0)
  if (dm.D == 128 && dm.P == 16) QUEST_FUSED(128, 16);
  else if (dm.D == 64 && dm.P == 8) QUEST_FUSED(64, 8);
  else if (dm.D == 64 && dm.P == 16) QUEST_FUSED(64, 16);
  else if (dm.D == 64 && dm.P == 32) QUEST_FUSED(64, 32);
  else if (dm.D == 64 && dm.P == 64) QUEST_FUSED(64, 64);
  else return hipErrorInvalidValue;
#undef QUEST_FUSED
#undef QUEST_FUSED_G
#undef QUEST_FUSED_A
  const hipError_t err = hipGetLastError();
  if (err != hipSuccess || plan.n_split == 1) return err;
  return launch_merge(dm, batch, plan, max_k, num_sel, workspace, out, stream,
                      xcd ? (int)(mblocks / kXcds) : 0);
}

hipError_t launch_decode_step(const Dims &dm, int batch, const void *q, const void *k_new,
                              const void *v_new, const int32_t *cu_new,
                              const int32_t *ctx_before, int max_new,
                              const int32_t *page_table, void *k_cache, void *v_cache,
                              void *kmeta, int reduce, const int32_t *ctx_lens,
                              const int32_t *budget_tokens, int max_k, int n_sink,
                              int n_recent, float sm_scale, float *scores,
                              int32_t *sel_pages, int32_t *num_sel, void *out,
                              float *workspace, hipStream_t stream) {
  const hipError_t err = launch_append_scores(dm, batch, q, k_new, v_new, cu_new, ctx_before,
                                              max_new, page_table, k_cache, v_cache, kmeta,
                                              reduce, scores, stream);
  if (err != hipSuccess) return err;
  return launch_topk_decode(dm, batch, q, k_cache, v_cache, page_table, ctx_lens, scores,
                            budget_tokens, max_k, n_sink, n_recent, sm_scale, sel_pages,
                            num_sel, out, workspace, stream);
}

}  // namespace quest
