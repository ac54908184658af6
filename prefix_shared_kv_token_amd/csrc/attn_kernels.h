// Device code of librdx for gfx950 (CDNA4): the prefix-shared attention
// kernels, the merge of split tiles, KV scatter and page-table writes.
// Included by exactly one translation unit (device.hip), which holds the
// host-side launch code.
//
// Attention follows the BatchLLM explainer, Horizontal Fusion section: the
// common-prefix part and each request's own part of prefix-shared attention
// are work of one kernel -- a row tile streams the shared-prefix keys and its
// requests' own keys, carrying one online-softmax state across both -- and
// when a tile's key ranges are split over several workgroups, their partial
// softmax states (o, running max m, running sum l) are combined with the
// log-sum-exp rule
//   M = max_c m_c,  w_c = l_c 2^(m_c - M),  o = sum_c w_c o_c / sum_c w_c
// (scores kept in the base-2 domain: t = s * scale * log2 e) by a merge pass
// queued right behind the attention kernel.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <vector>

#include "common.h"
#include "plan.h"

namespace rdx {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kThreads = 256;  // 4 waves of 64; wave w owns tile rows [32w, 32w+32)

struct AttnArgs {
  const int32_t* items;
  const int32_t* tiles;
  const int32_t* jobs;
  const int32_t* toks;
  const int32_t* contribs;
  const int32_t* cptr;
  const int32_t* clist;
  const int32_t* mblocks;
  const int32_t* page_table;
  int64_t ld;
  const void* q;
  const void* kp;
  const void* vp;
  void* o;
  float* ws_o;
  float* ws_ml;
  int64_t ws_tokens;
  int64_t pool_bytes;  // bytes of each KV pool
  int32_t row_bytes;   // bytes from one slot's row of a pool to the next
  int hq, hkv, group;
  float scale_log2;  // softmax scale * log2(e)
};

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ void store_out(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_out(__bf16* p, float v) { *p = (__bf16)v; }

// ---------------------------------------------------------------------------
// Merge of split tiles.  A contribution's partial for (tile token t, grouped
// head hh) lives at
//   ws_o [((kvh * ws_tokens + base + t - lo) * group + hh) * D + d]
//   ws_ml[((kvh * ws_tokens + base + t - lo) * group + hh) * 2 + {0: m, 1: l}]
// with o already normalised by its own l.  Each workgroup merges 16 query
// rows of one split tile for one KV head (16 lanes per row, D/16 values per
// lane), visiting only the partials that cover the row's token (the plan
// lists their workspace tokens per tile token).  It runs after the attention
// kernel in stream order.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void merge_kernel(AttnArgs a) {
  constexpr int kPer = D / 16;  // values per lane
  constexpr int kV4 = kPer / 4;
  // merge block record: first row, tile token count, tile first token, the
  // block's first tile token and its tokens' merge-list offsets (no tile or
  // offset lookups); merge-list entries are workspace tokens
  const int32_t* mb = a.mblocks + (int64_t)(blockIdx.x / a.hkv) * kMBlockWords;
  const int kvh = blockIdx.x % a.hkv;
  const int group = a.group;
  const int row = mb[0] + threadIdx.x / 16;
  const int part = threadIdx.x % 16;
  const bool live = row < mb[1] * group;  // 16-lane groups stay whole for the shuffles
  const int t = live ? row / group : 0, hh = live ? row % group : 0;
  const int lt = live ? t - mb[3] : 0;
  const int cs = live ? mb[4 + lt] : 0, n = live ? mb[5 + lt] - cs : 0;
  const int32_t q_index = live ? a.toks[(int64_t)(mb[2] + t) * kTokWords] : 0;
  const int rbase = kvh * (int)a.ws_tokens;
  float acc[kPer];
#pragma unroll
  for (int e = 0; e < kPer; ++e) acc[e] = 0.f;
  float wsum = 0.f, mrun = -INFINITY;
  // partials in batches of 16: once the list entries are in, lane `part`
  // reads (m, l) of one partial while every lane reads its slice of o of all
  // of them -- one round trip -- and then the weights are formed and applied
  for (int k0 = 0; k0 < n; k0 += 16) {
    const int k = k0 + part;
    const int cnt = min(16, n - k0);
    int w = 0;
    if (k < n) w = (rbase + a.clist[cs + k]) * group + hh;
    float m = -INFINITY, l = 0.f;
    if (k < n) {
      m = a.ws_ml[(int64_t)w * 2];
      l = a.ws_ml[(int64_t)w * 2 + 1];
    }
    // only the partials this row has are read (lanes of rows with fewer
    // partials, or whole waves past every row's count, issue no load)
    float4 ov[16][kV4];
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const int wj = __shfl(w, j, 16);
      const float4* src = reinterpret_cast<const float4*>(a.ws_o + (int64_t)wj * D + part * kPer);
#pragma unroll
      for (int e = 0; e < kV4; ++e) ov[j][e] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j < cnt) {
#pragma unroll
        for (int e = 0; e < kV4; ++e) ov[j][e] = src[e];
      }
    }
    float bm = l > 0.f ? m : -INFINITY;
#pragma unroll
    for (int o = 8; o > 0; o >>= 1) bm = fmaxf(bm, __shfl_xor(bm, o, 16));
    const float mnew = fmaxf(mrun, bm);
    if (mrun != -INFINITY && mnew != mrun) {
      const float sc = exp2_fast(mrun - mnew);
#pragma unroll
      for (int e = 0; e < kPer; ++e) acc[e] *= sc;
      wsum *= sc;
    }
    mrun = mnew;
    const float wt = l > 0.f ? l * exp2_fast(m - mnew) : 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
      const float wj = __shfl(wt, j, 16);
#pragma unroll
      for (int e = 0; e < kV4; ++e) {
        acc[4 * e] += wj * ov[j][e].x;
        acc[4 * e + 1] += wj * ov[j][e].y;
        acc[4 * e + 2] += wj * ov[j][e].z;
        acc[4 * e + 3] += wj * ov[j][e].w;
      }
      wsum += wj;
    }
  }
  if (!live) return;
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  T* dst = reinterpret_cast<T*>(a.o) + ((int64_t)q_index * a.hq + (int64_t)kvh * group + hh) * D + part * kPer;
#pragma unroll
  for (int e = 0; e < kPer; ++e) store_out(dst + e, acc[e] * inv);
}

// ---------------------------------------------------------------------------
// Iteration over the 64-key blocks of a work item's jobs.
// ---------------------------------------------------------------------------
struct BlockIter {
  int j, kb, k1;
  const int32_t* prow;
};

__device__ __forceinline__ void iter_job(const AttnArgs& a, BlockIter& it, int j) {
  const int32_t* job = a.jobs + (int64_t)j * kJobWords;
  it.j = j;
  it.prow = a.page_table + (int64_t)job[0] * a.ld;
  it.kb = job[1];
  it.k1 = job[2];
}

__device__ __forceinline__ void iter_next(const AttnArgs& a, BlockIter& it, int je) {
  it.kb += 64;
  if (it.kb >= it.k1 && it.j + 1 < je) iter_job(a, it, it.j + 1);
}

// Slot of key `i` of the block.  Positions past the job's end read the
// job's last position instead (a valid slot); those keys are masked out of
// the softmax, so their K/V rows only cost bandwidth.
__device__ __forceinline__ int block_slot(const BlockIter& it, int i) {
  return it.prow[min(it.kb + i, it.k1 - 1)];
}

// ---------------------------------------------------------------------------
// K/V tile staging helpers (4 key rows x one 16-byte chunk per unit)
// ---------------------------------------------------------------------------
struct Rows4 {
  uint4 a, b, c, d;
};

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// Reads 16-byte chunks of pool rows.  OFF32: the pool is under 2 GiB and is
// addressed through a raw buffer resource with 32-bit byte offsets
// (slot * row_bytes + chunk offset, a 24-bit multiply since such a pool has
// fewer than 2^24 rows of at least 128 bytes; the offset 2^31 is past its end,
// so a load there returns zeros); otherwise 64-bit pointer arithmetic.
template <bool OFF32>
struct PoolReader {
  __amdgpu_buffer_rsrc_t rsrc;
  const char* base;
  uint32_t row_bytes;
  __device__ void init(const void* pool, int64_t pool_bytes, uint32_t rb) {
    base = reinterpret_cast<const char*>(pool);
    row_bytes = rb;
    if constexpr (OFF32) rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(pool), (short)0, (int)pool_bytes, 0x00020000);
  }
  __device__ __forceinline__ uint4 chunk(int slot, uint32_t off) const {
    if constexpr (OFF32) {
      const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)(__umul24((uint32_t)slot, row_bytes) + off), 0, 0);
      return make_uint4(v.x, v.y, v.z, v.w);
    } else {
      return *reinterpret_cast<const uint4*>(base + (int64_t)slot * row_bytes + off);
    }
  }
  __device__ __forceinline__ Rows4 rows(const int4& s, uint32_t off) const {
    Rows4 r;
    r.a = chunk(s.x, off);
    r.b = chunk(s.y, off);
    r.c = chunk(s.z, off);
    r.d = chunk(s.w, off);
    return r;
  }
  // valid == false: no row is wanted (the slots may be stale or never
  // written).  With 32-bit offsets the loads get an offset past the buffer's
  // end and return zeros without a memory access; otherwise they read row 0,
  // which always exists.
  __device__ __forceinline__ Rows4 rows_if(const int4& s, uint32_t off, bool valid) const {
    if constexpr (OFF32) {
      auto o = [&](int slot) { return valid ? __umul24((uint32_t)slot, row_bytes) + off : 0x80000000u; };
      auto ld = [&](uint32_t x) {
        const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(rsrc, (int)x, 0, 0);
        return make_uint4(v.x, v.y, v.z, v.w);
      };
      Rows4 r;
      r.a = ld(o(s.x));
      r.b = ld(o(s.y));
      r.c = ld(o(s.z));
      r.d = ld(o(s.w));
      return r;
    } else {
      return rows(valid ? s : make_int4(0, 0, 0, 0), off);
    }
  }
};

template <int D>
__device__ __forceinline__ void store_k_rows(__bf16* k, const Rows4& r, int qd, int cc) {
  constexpr int KS = D + 8;
  __bf16* p = k + (4 * qd) * KS + 8 * cc;
  *reinterpret_cast<uint4*>(p) = r.a;
  *reinterpret_cast<uint4*>(p + KS) = r.b;
  *reinterpret_cast<uint4*>(p + 2 * KS) = r.c;
  *reinterpret_cast<uint4*>(p + 3 * KS) = r.d;
}

// V^T column of key quad qd: quads are stored in the MFMA contraction order
// (within each 16 keys: quads 0, 2, 1, 3)
__device__ __forceinline__ int vt_col(int qd) {
  const int qk = qd & 3;
  return 16 * (qd >> 2) + 4 * (qk == 1 ? 2 : (qk == 2 ? 1 : qk));
}

// 4 keys x 8 d of V -> 8 rows (d = 8 cc ..) x 4 keys of V^T
__device__ __forceinline__ void vt_pair(__bf16* vt, int vs, int d, int col, uint32_t w0, uint32_t w1, uint32_t w2,
                                        uint32_t w3) {
  // low halves of (w0, w1) and (w2, w3) -> row d; high halves -> row d + 1
  const uint2 lo2 = make_uint2(__builtin_amdgcn_perm(w1, w0, 0x05040100u), __builtin_amdgcn_perm(w3, w2, 0x05040100u));
  const uint2 hi2 = make_uint2(__builtin_amdgcn_perm(w1, w0, 0x07060302u), __builtin_amdgcn_perm(w3, w2, 0x07060302u));
  *reinterpret_cast<uint2*>(vt + d * vs + col) = lo2;
  *reinterpret_cast<uint2*>(vt + (d + 1) * vs + col) = hi2;
}

template <int D>
__device__ __forceinline__ void store_vt_rows(__bf16* vt, const Rows4& r, int cc, int col) {
  constexpr int VS = 64 + 8;
  const int d = 8 * cc;
  vt_pair(vt, VS, d, col, r.a.x, r.b.x, r.c.x, r.d.x);
  vt_pair(vt, VS, d + 2, col, r.a.y, r.b.y, r.c.y, r.d.y);
  vt_pair(vt, VS, d + 4, col, r.a.z, r.b.z, r.c.z, r.d.z);
  vt_pair(vt, VS, d + 6, col, r.a.w, r.b.w, r.c.w, r.d.w);
}

// ---------------------------------------------------------------------------
// bf16 kernel.  One workgroup per work item (tile, KV head, key ranges).
// Wave w holds query rows 32w..32w+31 of the tile; lane (i = lane % 32,
// h = lane / 32).  Scores are computed transposed, S^T = K Q^T, with the
// 32x32x16 bf16 MFMA so that each lane owns one query column: the row max is
// a reduction over the lane's registers plus one exchange with lane ^ 32, and
// the probabilities feed the P.V MFMA (O^T = V^T P^T) straight from
// registers.  The contraction order inside a 16-key step is permuted
// identically on both operands: lane half h holds keys {4h..4h+3, 8+4h..
// 8+4h+3}; V^T is stored in LDS with its key quads in that order.
//
// Pipeline: page-table slots are fetched two key blocks ahead and K/V rows
// one block ahead into registers while the MFMAs of the current block run;
// K and V^T live in a double-buffered LDS tile, one barrier per block.
// ---------------------------------------------------------------------------
template <int D>
struct KVTile {
  static constexpr int KS = D + 8;   // K tile row stride (elements), padded
  static constexpr int VS = 64 + 8;  // V^T tile row stride
  __bf16 k[64 * KS];
  __bf16 vt[D * VS];
};

// max(x, x of lane ^ 32) via the gfx950 half-wave swap (a VALU op, no LDS)
__device__ __forceinline__ float half_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Scheduling hint for a run of N (LDS operand read, MFMA) pairs: issue
// four reads first, then alternate one MFMA / one read, then the last four
// MFMAs, so each MFMA finds its operand already loaded.
template <int N>
__device__ __forceinline__ void sched_lds_mfma() {
  constexpr int kDsRead = 0x100, kMfma = 0x008;
  __builtin_amdgcn_sched_group_barrier(kDsRead, 4, 0);
#pragma unroll
  for (int i = 0; i < N - 4; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kDsRead, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kMfma, 4, 0);
}

// S^T = K Q^T for the 64 keys of tile t x this wave's 32 queries.  The two
// 32-key halves are interleaved (independent accumulators) and the
// scheduler is told to keep LDS operand reads several MFMAs ahead.
template <int D>
__device__ __forceinline__ void wave_scores(const KVTile<D>& t, const bf16x8 (&qreg)[D / 16], f32x16 (&s)[2], int li,
                                            int hi) {
  constexpr int KS = KVTile<D>::KS;
  constexpr int KSTEPS = D / 16;
  s[0] = f32x16{};
  s[1] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks)
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&t.k[(32 * kb2 + li) * KS + 16 * ks + 8 * hi]);
      s[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[ks], s[kb2], 0, 0, 0);
    }
  sched_lds_mfma<2 * KSTEPS>();
}

// The rest of a block once its scores s are in: mask (block-local keys >=
// rel are invisible to this lane's row), online softmax in base 2 with lazy
// rescale, O^T += V^T P^T from tile t.
template <int D>
__device__ __forceinline__ void wave_update(const KVTile<D>& t, f32x16 (&s)[2], f32x16 (&acc)[D / 32], float& m_run,
                                            float& l_run, int rel, float c2, int li, int hi) {
  constexpr int VS = KVTile<D>::VS;
  constexpr int DB = D / 32;
  // mask (only where some lane of the wave needs it) + online softmax, base 2
    if (__ballot(rel < 64)) {
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kl = 32 * kb2 + 8 * (r >> 2) + 4 * hi + (r & 3);
        s[kb2][r] = kl < rel ? s[kb2][r] : -INFINITY;
      }
  }
  // row max: four independent chains, then the other half-wave via permlane32 swap
  float mxp[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
    for (int r = 0; r < 16; ++r) mxp[r & 3] = fmaxf(mxp[r & 3], s[kb2][r]);
  float mx = fmaxf(fmaxf(mxp[0], mxp[1]), fmaxf(mxp[2], mxp[3]));
  mx = half_swap_max(mx);
  // Lazy rescale: the running max moves only when a score exceeds it by
  // more than 2^8, so probabilities stay <= 256 (exact: the same stale
  // max scales numerator and denominator) and most blocks skip the
  // O rescale.
  const float t_max = mx * c2;
  const float m_new = t_max > m_run + 8.f ? t_max : m_run;
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = exp2_fast(m_run - m_use);
  float lsp[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2_fast(fmaf(s[kb2][r], c2, -m_use));
      s[kb2][r] = p;
      lsp[r & 3] += p;
    }
  const float lsum = (lsp[0] + lsp[1]) + (lsp[2] + lsp[3]);
  l_run = l_run * alpha + lsum;
  m_run = m_new;
  if (__ballot(alpha != 1.f)) {
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[db][r] *= alpha;
  }
  // P (B operand): 16-key step ks uses registers 8t..8t+7 of block ks/2
  bf16x8 pk[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int e = 0; e < 8; ++e) pk[ks][e] = (__bf16)s[ks >> 1][8 * (ks & 1) + e];
  // O^T += V^T P^T (d blocks interleaved: independent accumulators)
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const bf16x8 va = *reinterpret_cast<const bf16x8*>(&t.vt[(32 * db + li) * VS + 16 * ks + 8 * hi]);
      acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pk[ks], acc[db], 0, 0, 0);
    }
  sched_lds_mfma<4 * DB>();
}

// One 64-key block for one wave's 32 query rows: scores, then update.
template <int D>
__device__ __forceinline__ void wave_block(const KVTile<D>& t, const bf16x8 (&qreg)[D / 16], f32x16 (&acc)[D / 32],
                                           float& m_run, float& l_run, int rel, float c2, int li, int hi) {
  f32x16 s[2];
  wave_scores<D>(t, qreg, s, li, hi);
  wave_update<D>(t, s, acc, m_run, l_run, rel, c2, li, hi);
}

// Final result of one lane's row: the normalised output (direct tiles; its
// caller Q/O row q_index) or the partial state (split tiles: the item's
// contribution covers tile tokens [act_lo, act_hi) at workspace token
// ws_base).
template <int D>
__device__ __forceinline__ void write_result(const AttnArgs& a, bool split, int act_lo, int act_hi, int ws_base,
                                             int32_t q_index, int kvh, const f32x16 (&acc)[D / 32], float m_run,
                                             float l_run, bool row_ok, int tloc, int row, int hi) {
  constexpr int DB = D / 32;
  const int group = a.group;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (!split) {
    // Lane (row, hi) holds d = 32 db + 8 g4 + 4 hi + (0..3).  Pairs of
    // 4-value pieces are exchanged with lane ^ 32 (v_permlane32_swap), so
    // each lane stores whole 16-byte runs: hi = 0 the 8 values of g4 = 2p,
    // hi = 1 those of g4 = 2p + 1 (half the store instructions).
    __bf16* dst = reinterpret_cast<__bf16*>(a.o) + ((int64_t)q_index * a.hq + (int64_t)kvh * group + row % group) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        bf16x4 v0, v1;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v0[e] = (__bf16)(acc[db][8 * p + e] * inv);
          v1[e] = (__bf16)(acc[db][8 * p + 4 + e] * inv);
        }
        const u32x2 w0 = __builtin_bit_cast(u32x2, v0), w1 = __builtin_bit_cast(u32x2, v1);
        const auto x = __builtin_amdgcn_permlane32_swap(w0.x, w1.x, false, false);
        const auto y = __builtin_amdgcn_permlane32_swap(w0.y, w1.y, false, false);
        // hi = 0: its own piece of g4 = 2p, then its partner's; hi = 1: its
        // partner's piece of g4 = 2p + 1, then its own
        const u32x4 out = u32x4{x[0], y[0], x[1], y[1]};
        if (row_ok) *reinterpret_cast<u32x4*>(dst + 32 * db + 16 * p + 8 * hi) = out;
      }
    return;
  }
  if (row_ok && tloc >= act_lo && tloc < act_hi) {
    const int64_t w = ((int64_t)kvh * a.ws_tokens + ws_base + tloc - act_lo) * group + row % group;
    float* dst = a.ws_o + w * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4)
        *reinterpret_cast<float4*>(dst + 32 * db + 8 * g4 + 4 * hi) =
            make_float4(acc[db][4 * g4] * inv, acc[db][4 * g4 + 1] * inv, acc[db][4 * g4 + 2] * inv,
                        acc[db][4 * g4 + 3] * inv);
    if (hi == 0) {
      a.ws_ml[w * 2] = m_run;
      a.ws_ml[w * 2 + 1] = l_tot;
    }
  }
}

template <int D, bool OFF32>
__global__ __launch_bounds__(kThreads, 2) void attn_bf16_kernel(AttnArgs a) {
  __shared__ KVTile<D> buf[2];
  __shared__ int4 slot_buf[2][16];  // page-table slots of the next two key blocks
  constexpr int KSTEPS = D / 16;  // MFMA k-steps over head_dim
  constexpr int DB = D / 32;      // 32-wide d blocks of the output
  constexpr int CH = D / 8;       // 16-byte chunks per K/V row
  constexpr int UNITS = 16 * CH;  // (key quad, chunk) units per matrix
  constexpr bool BOTH = 2 * UNITS > kThreads;  // each thread loads K and V of one unit

  // Load units: a unit is (key quad qd, 16-byte chunk cc) of the 64 x D tile.
  // K units vary cc fastest (16 lanes read one contiguous key row; row-major
  // LDS stores).  V units vary qd fastest so that 16 consecutive lanes store
  // 16 different 8-byte key quads of one V^T row (no LDS bank conflicts).
  // head_dim 128: every thread loads one K and one V unit; 64: threads
  // 0..127 load K, 128..255 load V (wave-uniform).
  const int tid = threadIdx.x;
  const bool doK = BOTH || tid < UNITS;  // (otherwise the thread loads V)
  const int uk = tid % UNITS;
  const int uv = BOTH ? tid : tid - UNITS;
  const int qd_k = uk / CH, cc_k = uk % CH;
  const int qd_v = uv % 16, cc_v = uv / 16;
  const int qd1 = doK ? qd_k : qd_v;  // the unit whose slots feed kr (head_dim 64: this thread's only unit)

  // one item record per key chunk, run for every KV head: workgroup b takes
  // record b / Hkv and KV head b % Hkv
  const int32_t* item = a.items + (int64_t)(blockIdx.x / (unsigned)a.hkv) * kItemWords;
  const int32_t* tile = a.tiles + (int64_t)item[0] * kTileWords;
  const int kvh = (int)(blockIdx.x % (unsigned)a.hkv);
  const int jb = item[1], je = item[2];
  const int tok_begin = tile[0], n_tok = tile[1];
  const int group = a.group;
  const int n_rows = n_tok * group;
  const int lane = tid & 63, wave = tid >> 6;
  const int li = lane & 31, hi = lane >> 5;
  const int row = wave * 32 + li;  // this lane's query row in the tile
  const int tloc = row / group;    // tile-local token
  // tokens this item attends for: all of a direct tile, the contribution's
  // range of a split tile
  int act_lo = 0, act_hi = n_tok;
  if (tile[4] >= 0) {
    const int32_t* cr0 = a.contribs + (int64_t)(tile[3] + item[3]) * kContribWords;
    act_lo = cr0[0];
    act_hi = cr0[1];
  }
  const bool row_ok = row < n_rows && tloc >= act_lo && tloc < act_hi;
  const bool wave_live = __ballot(row_ok) != 0;

  // ---- Q (B operand): Q[row][16 ks + 8 h .. +8) ----
  bf16x8 qreg[KSTEPS];
  int qpos = 0;
  {
    const __bf16* q = reinterpret_cast<const __bf16*>(a.q);
    if (row_ok) {
      const int32_t* tk = a.toks + (int64_t)(tok_begin + tloc) * kTokWords;
      qpos = tk[1];
      const __bf16* src = q + ((int64_t)tk[0] * a.hq + (int64_t)kvh * group + row % group) * D + 8 * hi;
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(src + 16 * s);
    } else {
#pragma unroll
      for (int s = 0; s < KSTEPS; ++s) qreg[s] = bf16x8{};
    }
  }

  f32x16 acc[DB];
#pragma unroll
  for (int b = 0; b < DB; ++b) acc[b] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = a.scale_log2;

  const uint32_t row_bytes = (uint32_t)a.row_bytes;
  PoolReader<OFF32> kpool, vpool;
  kpool.init(a.kp, a.pool_bytes, row_bytes);
  vpool.init(a.vp, a.pool_bytes, row_bytes);
  const uint32_t off1 = (uint32_t)(kvh * D + 8 * (doK ? cc_k : cc_v)) * 2;
  const uint32_t off2 = (uint32_t)(kvh * D + 8 * cc_v) * 2;

  int nblk = 0;
  for (int j = jb; j < je; ++j) {
    const int32_t* job = a.jobs + (int64_t)j * kJobWords;
    nblk += (job[2] - job[1] + 63) >> 6;
  }

  // r1: rows of the thread's first unit (K; head_dim 64: K or V, whichever
  // this thread loads); r2: rows of its V unit (head_dim 128 only).
  Rows4 r1, r2;
  const PoolReader<OFF32>& pool1 = doK ? kpool : vpool;
  auto load_kv = [&](const int4 (&sb)[16]) {
    r1 = pool1.rows(sb[qd1], off1);
    if constexpr (BOTH) r2 = vpool.rows(sb[qd_v], off2);
  };
  const int vcol = vt_col(qd_v);
  auto store_kv = [&](KVTile<D>& t) {
    if constexpr (BOTH) {
      store_k_rows<D>(t.k, r1, qd_k, cc_k);
      store_vt_rows<D>(t.vt, r2, cc_v, vcol);
    } else if (doK) {
      store_k_rows<D>(t.k, r1, qd_k, cc_k);
    } else {
      store_vt_rows<D>(t.vt, r1, cc_v, vcol);
    }
  };
  int* slot_words = reinterpret_cast<int*>(&slot_buf[0][0]);

  if (nblk > 0) {
    // ---- prologue: slots of blocks 0 and 1 into LDS, block 0 into LDS ----
    BlockIter it_slot, it_comp;
    iter_job(a, it_slot, jb);
    it_comp = it_slot;
    if (tid < 64) slot_words[tid] = block_slot(it_slot, tid);
    iter_next(a, it_slot, je);
    if (nblk > 1) {
      if (tid < 64) slot_words[64 + tid] = block_slot(it_slot, tid);
      iter_next(a, it_slot, je);
    }
    __syncthreads();
    load_kv(slot_buf[0]);
    store_kv(buf[0]);
    __syncthreads();

    int cur_job = -1, lim = 0;
    bool wave_job = false;
    for (int b = 0; b < nblk; ++b) {
      // ---- issue the K/V loads of block b+1 and the page-table read of block b+2 ----
      if (b + 1 < nblk) load_kv(slot_buf[(b + 1) & 1]);
      int slot_after = 0;
      const bool more = b + 2 < nblk;
      if (more) {
        if (tid < 64) slot_after = block_slot(it_slot, tid);
        iter_next(a, it_slot, je);
      }
      // ---- compute block b ----
      if (it_comp.j != cur_job) {
        cur_job = it_comp.j;
        const int32_t* job = a.jobs + (int64_t)cur_job * kJobWords;
        const int k1 = job[2], lo = job[3], hi_t = job[4], causal = job[5];
        lim = (row_ok && tloc >= lo && tloc < hi_t) ? (causal ? min(k1, qpos + 1) : k1) : 0;
        wave_job = wave_live && __ballot(lim > job[1]) != 0;
      }
      const KVTile<D>& t = buf[b & 1];
      if (wave_job) {
        wave_block<D>(t, qreg, acc, m_run, l_run, lim - it_comp.kb, c2, li, hi);
      }
      // ---- block b+1 into the other buffer ----
      if (b + 1 < nblk) store_kv(buf[(b + 1) & 1]);
      if (more && tid < 64) slot_words[(b & 1) * 64 + tid] = slot_after;
      iter_next(a, it_comp, je);
      __syncthreads();
    }
  }

  const int32_t q_index = row_ok ? a.toks[(int64_t)(tok_begin + tloc) * kTokWords] : 0;
  write_result<D>(a, item[7] >= 0, item[8], item[9], item[10], q_index, kvh, acc, m_run, l_run, row_ok, tloc, row, hi);
}

// ---------------------------------------------------------------------------
// bf16 decode kernel: tiles of at most 64 query rows (decode tiles are a
// sharing group's new tokens x the GQA group, which fit), one workgroup per
// work item.  Memory-bound by design, so it is built to keep many bytes in
// flight: each thread stages 1/256 of a 64-key K and V block (4 threads per
// key row) and two blocks are in flight in registers while a third is being
// computed from LDS.  Wave w owns rows 16w..16w+15 and uses the 16x16x32 bf16
// MFMA: S^T = K Q^T (K read row-major from LDS), then O^T = V^T P^T with V^T
// fragments from the gfx950 transposing LDS read (ds_read_b64_tr_b16) of the
// row-major V block; P^T is the score accumulator repacked to bf16 in place,
// with the keys of each 32-key step taken in the order the accumulators hold
// them (lane group g: keys 4g..4g+3 of the first 16, then of the second).
// Keys past a job's end and blocks past the item's end are loaded through
// out-of-range buffer offsets, which return zeros without touching memory.
// ---------------------------------------------------------------------------
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

template <int D>
struct DecTile {
  static constexpr int KS = D + 8;   // K row stride (elements): conflict-free 16-byte fragment reads
  static constexpr int VS = D + 16;  // V row stride: conflict-free transposing reads
  __bf16 k[64 * KS];
  __bf16 v[64 * VS];
};

// max / sum of x over lanes l and l ^ 16 (gfx950 row swap, no LDS)
__device__ __forceinline__ float row16_swap_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float row16_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float half_swap_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

constexpr uint32_t kNoRow = 0x80000000u;  // buffer offset past any pool this path addresses

// One thread's share of a K/V block: CPT 16-byte chunks of one key row of K
// and of V.
template <int CPT>
struct DecStage {
  uint4 k[CPT], v[CPT];
};

template <int D, bool OFF32>
struct DecPool {
  __amdgpu_buffer_rsrc_t kr, vr;
  const char *kb, *vb;
  uint32_t row_bytes;
  __device__ void init(const AttnArgs& a) {
    row_bytes = (uint32_t)a.row_bytes;
    kb = reinterpret_cast<const char*>(a.kp);
    vb = reinterpret_cast<const char*>(a.vp);
    if constexpr (OFF32) {
      kr = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.kp), (short)0, (int)a.pool_bytes, 0x00020000);
      vr = __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(a.vp), (short)0, (int)a.pool_bytes, 0x00020000);
    }
  }
  // byte offset of this thread's first chunk for `slot` (< 0: no row).
  // 64-bit path: the slot itself, -1 for no row.
  __device__ __forceinline__ uint32_t offset(int slot, uint32_t in_row) const {
    if constexpr (OFF32) return slot >= 0 ? __umul24((uint32_t)slot, row_bytes) + in_row : kNoRow;
    else return (uint32_t)slot;
  }
  template <int CPT>
  __device__ __forceinline__ void load(DecStage<CPT>& st, uint32_t o, uint32_t in_row) const {
    // 64-bit path, no row: the load still goes out (to row 0, which always
    // exists: no branch around the load) and the staged values are zeros, so
    // the masked key's V row enters P.V as 0 whatever row 0 holds
    const bool none = !OFF32 && (int)o < 0;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
      if constexpr (OFF32) {
        const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(kr, (int)(o + 16 * i), 0, 0);
        const u32x4 y = __builtin_amdgcn_raw_buffer_load_b128(vr, (int)(o + 16 * i), 0, 0);
        st.k[i] = make_uint4(x.x, x.y, x.z, x.w);
        st.v[i] = make_uint4(y.x, y.y, y.z, y.w);
      } else {
        const int64_t off = (int64_t)(none ? 0u : o) * row_bytes + in_row + 16 * i;
        const uint4 x = *reinterpret_cast<const uint4*>(kb + off);
        const uint4 y = *reinterpret_cast<const uint4*>(vb + off);
        // zeros by a mask, not a select of the two vectors (which the
        // compiler lowers through private memory)
        const uint32_t keep = none ? 0u : ~0u;
        st.k[i] = make_uint4(x.x & keep, x.y & keep, x.z & keep, x.w & keep);
        st.v[i] = make_uint4(y.x & keep, y.y & keep, y.z & keep, y.w & keep);
      }
    }
  }
};

template <int D, int CPT>
__device__ __forceinline__ void dec_store(DecTile<D>& t, const DecStage<CPT>& st, int kk, int cq) {
  __bf16* kp = t.k + kk * DecTile<D>::KS + 8 * CPT * cq;
  __bf16* vp = t.v + kk * DecTile<D>::VS + 8 * CPT * cq;
#pragma unroll
  for (int i = 0; i < CPT; ++i) {
    *reinterpret_cast<uint4*>(kp + 8 * i) = st.k[i];
    *reinterpret_cast<uint4*>(vp + 8 * i) = st.v[i];
  }
}

// One 64-key block for one wave's 16 rows (lane: row rr = lane % 16, lane
// group g = lane / 16).  rel: block-local keys < rel are visible to the row.
template <int D>
__device__ __forceinline__ void dec_block(const DecTile<D>& t, const bf16x8 (&qf)[D / 32], f32x4 (&acc)[D / 16],
                                          float& m_run, float& l_run, int rel, float c2, int rr, int g) {
  constexpr int KS = DecTile<D>::KS, VS = DecTile<D>::VS;
  constexpr int DB = D / 32, DT = D / 16;
  f32x4 s[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) s[kt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int kt = 0; kt < 4; ++kt) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(&t.k[(16 * kt + rr) * KS + 32 * db + 8 * g]);
      s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qf[db], s[kt], 0, 0, 0);
    }
  if (__ballot(rel < 64)) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) s[kt][r] = 16 * kt + 4 * g + r < rel ? s[kt][r] : -INFINITY;
  }
  float mx = fmaxf(fmaxf(fmaxf(s[0][0], s[0][1]), fmaxf(s[0][2], s[0][3])),
                   fmaxf(fmaxf(s[1][0], s[1][1]), fmaxf(s[1][2], s[1][3])));
  mx = fmaxf(mx, fmaxf(fmaxf(fmaxf(s[2][0], s[2][1]), fmaxf(s[2][2], s[2][3])),
                       fmaxf(fmaxf(s[3][0], s[3][1]), fmaxf(s[3][2], s[3][3]))));
  mx = half_swap_max(row16_swap_max(mx));
  // lazy rescale (see wave_block)
  const float t_max = mx * c2;
  const float m_new = t_max > m_run + 8.f ? t_max : m_run;
  const float m_use = m_new == -INFINITY ? 0.f : m_new;
  const float alpha = exp2_fast(m_run - m_use);
  float lsp[4];
#pragma unroll
  for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
    for (int r = 0; r < 4; ++r) s[kt][r] = exp2_fast(fmaf(s[kt][r], c2, -m_use));
    lsp[kt] = (s[kt][0] + s[kt][1]) + (s[kt][2] + s[kt][3]);
  }
  // per-lane partial sum over this lane's keys (lanes of a row share m)
  l_run = l_run * alpha + ((lsp[0] + lsp[1]) + (lsp[2] + lsp[3]));
  m_run = m_new;
  if (__ballot(alpha != 1.f)) {
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
  }
  bf16x8 pk[2];
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pk[h][r] = (__bf16)s[2 * h][r];
      pk[h][4 + r] = (__bf16)s[2 * h + 1][r];
    }
  // O^T += V^T P^T: lane (rr, g) reads 8 bytes of V row 32h + 4g + rr/4 (and
  // +16) at column 16 dt + 4 (rr % 4); the transposing read hands it the
  // column rr of that 16 x 4 patch
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
#pragma unroll
  for (int h = 0; h < 2; ++h)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const __bf16* p0 = &t.v[(32 * h + 4 * g + (rr >> 2)) * VS + 16 * dt + 4 * (rr & 3)];
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0));
      const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(p0 + 16 * VS));
      // whole-word repack (element-wise extraction from the transposing
      // read's result is not lowered correctly by this compiler)
      const u32x2 lw = __builtin_bit_cast(u32x2, lo), hw = __builtin_bit_cast(u32x2, hi);
      const bf16x8 va = __builtin_bit_cast(bf16x8, u32x4{lw.x, lw.y, hw.x, hw.y});
      acc[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pk[h], acc[dt], 0, 0, 0);
    }
}

template <int D, bool OFF32>
__global__ __launch_bounds__(kThreads, 2) void attn_decode_kernel(AttnArgs a) {
  __shared__ DecTile<D> buf[2];
  constexpr int DB = D / 32, DT = D / 16;
  constexpr int CPT = D / 32;  // 16-byte chunks per thread: 4 threads per key row

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rr = lane & 15, g = lane >> 4;
  // the item record carries the tile, contribution and first-job fields, so
  // one read starts the page-table and Q loads (no tile/job/contribution
  // lookups on the way to the first K/V request)
  const int32_t* item = a.items + (int64_t)(blockIdx.x / (unsigned)a.hkv) * kItemWords;
  const int kvh = (int)(blockIdx.x % (unsigned)a.hkv);
  const int jb = item[1], je = item[2], nblk = item[4];
  const int tok_begin = item[5], n_tok = item[6];
  const bool split = item[7] >= 0;
  const int act_lo = item[8], act_hi = item[9], ws_base = item[10];
  const int group = a.group;
  const int n_rows = n_tok * group;
  const int row = 16 * wave + rr;
  const int tloc = row / group;
  const bool row_ok = row < n_rows && tloc >= act_lo && tloc < act_hi;
  const bool wave_live = __ballot(row_ok) != 0;

  // Q (B operand of S^T): Q[row][32 db + 8 g .. +8), loaded in the
  // prologue after the first K/V requests (below)
  bf16x8 qf[DB];
  int qpos = 0;
  f32x4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = a.scale_log2;

  DecPool<D, OFF32> pool;
  pool.init(a);
  const int kk = tid >> 2, cq = tid & 3;  // staging: key row kk, chunks CPT*cq ..
  const uint32_t in_row = (uint32_t)(kvh * D + 8 * CPT * cq) * 2;
  // slot of this thread's key in the block the iterator is at (-1: none)
  auto slot_of = [&](const BlockIter& it) { return it.kb + kk < it.k1 ? it.prow[it.kb + kk] : -1; };

  // the lane's token record (caller row, position); rows outside the tile
  // read their clamped token's: finite Q values whose keys are all masked and
  // whose results are never written
  const int tl = max(0, min(tloc, n_tok - 1));
  int2 tok = make_int2(0, 0);
  if (nblk > 0) {
    BlockIter it_s, it_c;
    it_s.j = jb;
    it_s.prow = a.page_table + (int64_t)item[11] * a.ld;
    it_s.kb = item[12];
    it_s.k1 = item[13];
    it_c = it_s;
    DecStage<CPT> r0, r1;
    // Loads retire in order for the wait counter: the page-table slots of
    // blocks 0-2 first, the token record behind them, then the K/V of blocks
    // 0 and 1 (which wait for their slots only), and Q last, so no wait on
    // the way to the first K/V request includes the token record or Q.
    const int s0 = slot_of(it_s);
    iter_next(a, it_s, je);
    const int s1 = nblk > 1 ? slot_of(it_s) : -1;
    iter_next(a, it_s, je);
    int slot_next = nblk > 2 ? slot_of(it_s) : -1;  // block 2
    iter_next(a, it_s, je);
    tok = *reinterpret_cast<const int2*>(a.toks + (int64_t)(tok_begin + tl) * kTokWords);
    pool.load(r0, pool.offset(s0, in_row), in_row);
    pool.load(r1, pool.offset(s1, in_row), in_row);
    qpos = tok.y;
    {
      const __bf16* src = reinterpret_cast<const __bf16*>(a.q) +
                          ((int64_t)tok.x * a.hq + (int64_t)kvh * group + row % group) * D + 8 * g;
#pragma unroll
      for (int db = 0; db < DB; ++db) qf[db] = *reinterpret_cast<const bf16x8*>(src + 32 * db);
    }
    dec_store<D, CPT>(buf[0], r0, kk, cq);
    __syncthreads();

    // the first job's view from the item record
    int cur_job = jb;
    int lim = (row_ok && tloc >= item[14] && tloc < item[15]) ? (item[16] ? min(item[13], qpos + 1) : item[13]) : 0;
    bool wave_job = wave_live && __ballot(lim > item[12]) != 0;
    // block b: compute from buf[b & 1]; the registers of block b+1 are
    // stored behind it; block b+2 is issued into the registers block b used
    // Issue order matters (loads retire in order for the wait counter): the
    // page-table read for block b+3 goes out before the K/V loads of block
    // b+2, so the next step can wait for it without draining those loads.
    auto step = [&](int b, DecStage<CPT>& mine, DecStage<CPT>& next) {
      const int s2 = b + 2 < nblk ? slot_next : -1;
      slot_next = b + 3 < nblk ? slot_of(it_s) : -1;
      iter_next(a, it_s, je);
      pool.load(mine, pool.offset(s2, in_row), in_row);
      if (it_c.j != cur_job) {
        cur_job = it_c.j;
        const int32_t* job = a.jobs + (int64_t)cur_job * kJobWords;
        const int k1 = job[2], lo = job[3], hi_t = job[4], causal = job[5];
        lim = (row_ok && tloc >= lo && tloc < hi_t) ? (causal ? min(k1, qpos + 1) : k1) : 0;
        wave_job = wave_live && __ballot(lim > job[1]) != 0;
      }
      if (wave_job && b < nblk) dec_block<D>(buf[b & 1], qf, acc, m_run, l_run, lim - it_c.kb, c2, rr, g);
      dec_store<D, CPT>(buf[(b + 1) & 1], next, kk, cq);
      iter_next(a, it_c, je);
      __syncthreads();
    };
    // both half-steps unconditionally (a step past the last block only moves
    // zeros), so every loop trip leaves the same loads outstanding
    for (int b = 0; b < nblk; b += 2) {
      step(b, r0, r1);
      step(b + 1, r1, r0);
    }
  } else {
    tok = *reinterpret_cast<const int2*>(a.toks + (int64_t)(tok_begin + tl) * kTokWords);  // the output row
  }

  // ---- result: rows of this lane (4 lane groups share a row) ----
  const float l_tot = half_swap_sum(row16_swap_sum(l_run));
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (!split) {
    if (row_ok) {
      __bf16* dst = reinterpret_cast<__bf16*>(a.o) + ((int64_t)tok.x * a.hq + (int64_t)kvh * group + row % group) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = (__bf16)(acc[dt][r] * inv);
        *reinterpret_cast<bf16x4*>(dst + 16 * dt + 4 * g) = v;
      }
    }
    return;
  }
  if (row_ok) {  // row_ok implies act_lo <= tloc < act_hi
    const int64_t w = ((int64_t)kvh * a.ws_tokens + ws_base + tloc - act_lo) * group + row % group;
    float* dst = a.ws_o + w * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<float4*>(dst + 16 * dt + 4 * g) =
          make_float4(acc[dt][0] * inv, acc[dt][1] * inv, acc[dt][2] * inv, acc[dt][3] * inv);
    if (g == 0) {
      a.ws_ml[w * 2] = m_run;
      a.ws_ml[w * 2 + 1] = l_tot;
    }
  }
}

// ---------------------------------------------------------------------------
// Wide bf16 extend kernel (head_dim 128): 8 waves, 256-row tiles.  Each K/V
// block feeds twice the rows of the 4-wave kernel (half the loads, LDS stores
// and barriers per flop), and each thread stages only one unit (waves 0-3 K,
// waves 4-7 V).
//
// Ping-pong between the two waves of each SIMD (waves w and w+4): waves 0-3
// run block b as scores -> softmax -> P.V, waves 4-7 run softmax(b) -> P.V(b)
// -> scores(b+1), so one wave's MFMA runs line up with the other's softmax
// instead of both waves contending for the matrix core and then both idling
// it.  This needs block b+1 in LDS while block b is computed: three LDS
// buffers (block b, b+1, and b+2 being staged); K/V of block b+2 wait in
// registers while block b+3 is being loaded, and the page-table slots of block
// b+4 are read.
// ---------------------------------------------------------------------------
constexpr int kWideThreads = 512;

// Per-wave view of the job a key block belongs to.
struct JobView {
  int job = -1, lim = 0;
  bool live = false;  // some row of this wave attends to the job
};

__device__ __forceinline__ void job_view(const AttnArgs& a, const BlockIter& it, JobView& v, bool row_ok, int tloc,
                                         int qpos, bool wave_live) {
  if (it.j == v.job) return;
  v.job = it.j;
  const int32_t* job = a.jobs + (int64_t)it.j * kJobWords;
  const int k1 = job[2], lo = job[3], hi_t = job[4], causal = job[5];
  v.lim = (row_ok && tloc >= lo && tloc < hi_t) ? (causal ? min(k1, qpos + 1) : k1) : 0;
  v.live = wave_live && __ballot(v.lim > job[1]) != 0;
}

template <bool OFF32>
__global__ __launch_bounds__(kWideThreads, 1) void attn_bf16_wide_kernel(AttnArgs a) {
  constexpr int D = 128, KSTEPS = D / 16, DB = D / 32, CH = D / 8;
  __shared__ KVTile<D> buf[3];
  __shared__ int slot_ring[2][64];

  const int tid = threadIdx.x;
  // waves 0-3 stage K, 4-7 V; taken from lane 0 so the compiler sees a
  // wave-uniform choice (the pool's buffer resource stays in scalar registers)
  const bool doK = __builtin_amdgcn_readfirstlane(tid) < 256;
  const int u = tid & 255;
  const int qd = doK ? u / CH : u % 16;  // K units: chunk fastest; V units: key quad fastest
  const int cc = doK ? u % CH : u / 16;

  // one item record per key chunk, run for every KV head: workgroup b takes
  // record b / Hkv and KV head b % Hkv
  // everything the workgroup needs to start comes from its item record:
  // token range, contribution, block count, the first job and, when the
  // tile's caller rows are consecutive, its first Q row (the Q loads then
  // go out after this one read)
  const int32_t* item = a.items + (int64_t)(blockIdx.x / (unsigned)a.hkv) * kItemWords;
  const int kvh = (int)(blockIdx.x % (unsigned)a.hkv);
  const int jb = item[1], je = item[2], nblk = item[4];
  const int tok_begin = item[5], n_tok = item[6];
  const int act_lo = item[8], act_hi = item[9];
  const int group = a.group;
  const int n_rows = n_tok * group;
  const int lane = tid & 63, wave = tid >> 6;
  const bool ahead = wave >= 4;  // waves that compute scores one block ahead
  const int li = lane & 31, hi = lane >> 5;
  const int row = wave * 32 + li;
  const int tloc = row / group;
  const bool row_ok = row < n_rows && tloc >= act_lo && tloc < act_hi;
  const bool wave_live = __ballot(row_ok) != 0;

  // page-table slots of blocks 0-3, read first: loads retire in
  // order for the wait counter, so the slot-ring writes of the prologue wait
  // for these reads only, never for the K/V blocks or Q behind them
  BlockIter it_slot;
  it_slot.j = jb;
  it_slot.prow = a.page_table + (int64_t)item[11] * a.ld;
  it_slot.kb = item[12];
  it_slot.k1 = item[13];
  // (every wave reads them, without a lane condition, so no lane mask or
  // register merge forces an early wait; positions past the item's last
  // block read its last key's slot, which is valid)
  int sl[4] = {0, 0, 0, 0};
  if (nblk > 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sl[i] = block_slot(it_slot, lane);
      if (nblk > i) iter_next(a, it_slot, je);
    }
  }
  // the lane's token record (caller row, position), read right behind them
  const int tl = max(0, min(tloc, n_tok - 1));
  const int2 tok = *reinterpret_cast<const int2*>(a.toks + (int64_t)(tok_begin + tl) * kTokWords);

  // Q and the query position: loaded after the first K/V requests (below),
  // without a branch or a select on the loaded values, so no wait for a
  // page-table slot or a K/V block includes them.  Rows outside the tile's
  // active range read their clamped token's row: finite values whose keys
  // are all masked, and whose results are never written.
  bf16x8 qreg[KSTEPS];
  int qpos = 0;
  auto load_q = [&]() {
    const int32_t qi = item[17] >= 0 ? item[17] + tl : tok.x;
    qpos = tok.y;
    const __bf16* src = reinterpret_cast<const __bf16*>(a.q) +
                        ((int64_t)qi * a.hq + (int64_t)kvh * group + row % group) * D + 8 * hi;
#pragma unroll
    for (int s = 0; s < KSTEPS; ++s) qreg[s] = *reinterpret_cast<const bf16x8*>(src + 16 * s);
  };
  f32x16 acc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) acc[db] = f32x16{};
  float m_run = -INFINITY, l_run = 0.f;
  const float c2 = a.scale_log2;

  PoolReader<OFF32> pool;
  pool.init(doK ? a.kp : a.vp, a.pool_bytes, (uint32_t)a.row_bytes);
  const uint32_t off = (uint32_t)(kvh * D + 8 * cc) * 2;
  const int vcol = vt_col(qd);

  auto issue = [&](Rows4& r, const int* slots, bool valid = true) {
    const int4 sl = *reinterpret_cast<const int4*>(slots + 4 * qd);
    r = pool.rows_if(sl, off, valid);
  };
  auto stage = [&](KVTile<D>& t, const Rows4& r) {
    if (doK)
      store_k_rows<D>(t.k, r, qd, cc);
    else
      store_vt_rows<D>(t.vt, r, cc, vcol);
  };

  if (nblk > 0) {
    BlockIter it_comp, it_next;
    it_comp.j = jb;
    it_comp.prow = a.page_table + (int64_t)item[11] * a.ld;
    it_comp.kb = item[12];
    it_comp.k1 = item[13];
    Rows4 rA, rB;
    // ---- prologue: blocks 0 and 1 in LDS, block 2 loading, slots of block 3 in the ring ----
    if (tid < 64) {
      slot_ring[0][tid] = sl[0];
      slot_ring[1][tid] = sl[1];
    }
    __syncthreads();
    issue(rA, slot_ring[0]);
    if (nblk > 1) issue(rB, slot_ring[1]);
    load_q();
    __syncthreads();
    if (nblk > 2 && tid < 64) slot_ring[0][tid] = sl[2];
    stage(buf[0], rA);
    if (nblk > 1) stage(buf[1], rB);
    __syncthreads();
    if (nblk > 2) issue(rA, slot_ring[0]);
    if (nblk > 3 && tid < 64) slot_ring[1][tid] = sl[3];  // ring[1] was last read before the second barrier
    __syncthreads();

    JobView vc, vn;  // jobs of the block being finished and of the block after it
    it_next = it_comp;
    iter_next(a, it_next, je);
    f32x16 s[2];
    // the first job's view from the item record
    vc.job = jb;
    vc.lim = (row_ok && tloc >= item[14] && tloc < item[15]) ? (item[16] ? min(item[13], qpos + 1) : item[13]) : 0;
    vc.live = wave_live && __ballot(vc.lim > item[12]) != 0;
    if (ahead && vc.live) wave_scores<D>(buf[0], qreg, s, li, hi);

    int bc = 0;  // LDS buffer of block b
    // block b: rnext holds block b+2 (staged behind the compute), rcur is
    // reloaded with block b+3 from ring[(b+1) & 1]; the slots of block b+4 go
    // to ring[b & 1], which the previous step read.  Loads retire in order
    // for the wait counter, so the page-table read goes out before the K/V
    // loads, and nothing is loaded or staged under a branch (past the last
    // block the loads are out of range and the staged tile is never used):
    // each step then waits only for the block it stages.
    auto step = [&](int b, Rows4& rcur, Rows4& rnext) {
      const bool more = b + 4 < nblk;
      const int slot_after = block_slot(it_slot, tid & 63);  // clamped: always a valid position
      if (more) iter_next(a, it_slot, je);
      issue(rcur, slot_ring[(b + 1) & 1], b + 3 < nblk);
      const int bn = bc == 2 ? 0 : bc + 1, bs = bn == 2 ? 0 : bn + 1;
      if (b < nblk) {
        job_view(a, it_comp, vc, row_ok, tloc, qpos, wave_live);
        if (vc.live) {
          if (!ahead) wave_scores<D>(buf[bc], qreg, s, li, hi);
          wave_update<D>(buf[bc], s, acc, m_run, l_run, vc.lim - it_comp.kb, c2, li, hi);
        }
        if (ahead && b + 1 < nblk) {
          job_view(a, it_next, vn, row_ok, tloc, qpos, wave_live);
          if (vn.live) wave_scores<D>(buf[bn], qreg, s, li, hi);
        }
      }
      stage(buf[bs], rnext);
      if (more && tid < 64) slot_ring[b & 1][tid] = slot_after;
      iter_next(a, it_comp, je);
      iter_next(a, it_next, je);
      bc = bn;
      __syncthreads();
    };
    for (int b = 0; b < nblk; b += 2) {
      step(b, rB, rA);
      step(b + 1, rA, rB);
    }
  }
  const int32_t q_index = row_ok ? (item[17] >= 0 ? item[17] + tloc : tok.x) : 0;
  write_result<D>(a, item[7] >= 0, act_lo, act_hi, item[10], q_index, kvh, acc, m_run, l_run, row_ok, tloc, row, hi);
}

// ---------------------------------------------------------------------------
// fp32 kernel (plain VALU, parity-grade).  One thread per query row of the
// tile, scalar online softmax over the row's visible keys.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void attn_f32_kernel(AttnArgs a) {
  const int32_t* item = a.items + (int64_t)(blockIdx.x / (unsigned)a.hkv) * kItemWords;
  const int32_t* tile = a.tiles + (int64_t)item[0] * kTileWords;
  const int kvh = (int)(blockIdx.x % (unsigned)a.hkv);
  const int group = a.group;
  const int n_rows = tile[1] * group;
  const int row = threadIdx.x;
  if (row >= n_rows) return;
  const int tloc = row / group;
  float q[D], acc[D];
  float m_run = -INFINITY, l_run = 0.f;
  const int32_t* tk = a.toks + (int64_t)(tile[0] + tloc) * kTokWords;
  const int qpos = tk[1];
  const float* src = reinterpret_cast<const float*>(a.q) + ((int64_t)tk[0] * a.hq + (int64_t)kvh * group + row % group) * D;
  for (int d = 0; d < D; ++d) {
    q[d] = src[d];
    acc[d] = 0.f;
  }
  const float* kpool = reinterpret_cast<const float*>(a.kp);
  const float* vpool = reinterpret_cast<const float*>(a.vp);
  for (int j = item[1]; j < item[2]; ++j) {
    const int32_t* job = a.jobs + (int64_t)j * kJobWords;
    if (tloc < job[3] || tloc >= job[4]) continue;
    const int32_t* prow = a.page_table + (int64_t)job[0] * a.ld;
    const int end = job[5] ? min(job[2], qpos + 1) : job[2];
    for (int p = job[1]; p < end; ++p) {
      const int64_t off = (int64_t)prow[p] * (a.row_bytes / 4) + (int64_t)kvh * D;
      float s = 0.f;
      for (int d = 0; d < D; ++d) s = fmaf(q[d], kpool[off + d], s);
      const float t = s * a.scale_log2;
      const float m_new = fmaxf(m_run, t);
      const float alpha = exp2f(m_run - m_new);
      const float pw = exp2f(t - m_new);
      l_run = l_run * alpha + pw;
      for (int d = 0; d < D; ++d) acc[d] = fmaf(pw, vpool[off + d], acc[d] * alpha);
      m_run = m_new;
    }
  }
  const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
  if (tile[4] < 0) {
    float* dst = reinterpret_cast<float*>(a.o) + ((int64_t)tk[0] * a.hq + (int64_t)kvh * group + row % group) * D;
    for (int d = 0; d < D; ++d) dst[d] = acc[d] * inv;
    return;
  }
  const int32_t* cr = a.contribs + (int64_t)(tile[3] + item[3]) * kContribWords;
  if (tloc >= cr[0] && tloc < cr[1]) {
    const int64_t w = ((int64_t)kvh * a.ws_tokens + cr[2] + tloc - cr[0]) * group + row % group;
    for (int d = 0; d < D; ++d) a.ws_o[w * D + d] = acc[d] * inv;
    a.ws_ml[w * 2] = m_run;
    a.ws_ml[w * 2 + 1] = l_run;
  }
}

// ---------------------------------------------------------------------------
// KV scatter and page-table writes
// ---------------------------------------------------------------------------
// New rows arrive dense (row_vecs 16-byte vectors each); a pool row is
// pitch_vecs vectors apart.
__global__ void kv_store_kernel(uint4* __restrict__ kp, uint4* __restrict__ vp, const uint4* __restrict__ kn,
                                const uint4* __restrict__ vn, const int32_t* __restrict__ slots, int64_t n,
                                int64_t row_vecs, int64_t pitch_vecs) {
  const int64_t total = n * row_vecs;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t tok = i / row_vecs, e = i % row_vecs;
    const int64_t dst = (int64_t)slots[tok] * pitch_vecs + e;
    kp[dst] = kn[i];
    vp[dst] = vn[i];
  }
}

// Copies a staged work list from mapped pinned host memory to the device
// plan buffer (16 bytes per thread, grid-stride).  A kernel rather than a
// DMA copy: queued between kernels on one stream, a host-to-device DMA copy
// has stalled the stream for milliseconds at a time.
__global__ void plan_copy_kernel(const int4* __restrict__ src, int4* __restrict__ dst, int64_t n_vec4) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n_vec4; i += (int64_t)gridDim.x * blockDim.x)
    dst[i] = src[i];
}

__global__ void page_table_write_kernel(int32_t* __restrict__ pt, int64_t ld, const int32_t* __restrict__ runs,
                                        const int32_t* __restrict__ run_slots) {
  const int32_t* r = runs + (int64_t)blockIdx.x * kRunWords;
  int32_t* dst = pt + (int64_t)r[0] * ld + r[1];
  const int32_t* src = run_slots + r[3];
  for (int i = threadIdx.x; i < r[2]; i += blockDim.x) dst[i] = src[i];
}

// Everything one decode step must write before its attention launch, in one
// kernel: workgroups [0, n_copy) copy the work list from the mapped host
// staging buffer to the device plan buffer (16 bytes per thread), the next
// ceil(n_runs / 256) write the page-table runs (one per thread), the rest
// scatter the new K/V rows.
// Runs, run slots and new slots are read from the staging buffer too, since
// the device copy is being written by this same launch.
__global__ void step_store_kernel(const int4* __restrict__ stage, int4* __restrict__ dev_plan, int64_t n_vec4,
                                  int32_t n_copy, int32_t* __restrict__ pt, int64_t ld,
                                  const int32_t* __restrict__ runs, const int32_t* __restrict__ run_slots,
                                  int32_t n_runs, uint4* __restrict__ kp, uint4* __restrict__ vp,
                                  const uint4* __restrict__ kn, const uint4* __restrict__ vn,
                                  const int32_t* __restrict__ slots, int64_t n, int64_t row_vecs,
                                  int64_t pitch_vecs) {
  const int32_t bx = (int32_t)blockIdx.x;
  if (bx < n_copy) {
    for (int64_t i = (int64_t)bx * blockDim.x + threadIdx.x; i < n_vec4; i += (int64_t)n_copy * blockDim.x)
      dev_plan[i] = stage[i];
    return;
  }
  const int32_t n_pt = (n_runs + (int32_t)blockDim.x - 1) / (int32_t)blockDim.x;
  if (bx < n_copy + n_pt) {
    // one run per thread.  A decode step's runs are one entry each, in run
    // order, so the slot is read speculatively next to the run record (two
    // reads of mapped host memory in parallel instead of one after the
    // other) and used when the record confirms it.
    const int32_t ri = (bx - n_copy) * (int32_t)blockDim.x + (int32_t)threadIdx.x;
    if (ri >= n_runs) return;
    const int4 r = reinterpret_cast<const int4*>(runs)[ri];  // page row, first position, count, source
    const int32_t guess = run_slots[ri];  // in bounds: every run has at least one entry
    int32_t* dst = pt + (int64_t)r.x * ld + r.y;
    if (r.z == 1 && r.w == ri) {
      dst[0] = guess;
    } else {
      for (int i = 0; i < r.z; ++i) dst[i] = run_slots[r.w + i];
    }
    return;
  }
  const int64_t total = n * row_vecs;
  const int64_t nb = (int64_t)gridDim.x - n_copy - n_pt;
  for (int64_t i = ((int64_t)bx - n_copy - n_pt) * blockDim.x + threadIdx.x; i < total; i += nb * blockDim.x) {
    const int64_t tok = i / row_vecs, e = i % row_vecs;
    const int64_t dst = (int64_t)slots[tok] * pitch_vecs + e;
    kp[dst] = kn[i];
    vp[dst] = vn[i];
  }
}

}  // namespace rdx
