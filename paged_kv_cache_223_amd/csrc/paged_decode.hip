// Paged-KV decode attention for gfx950 (CDNA4).
//
// Method: "KV Cache Fragmentation" field guide (defragging.ai), section
// "Definition" — the cache is cut into fixed-size pages and the attention
// kernel walks the per-request table from logical to physical pages;
// "Paged Attention and KV Cache Fragmentation" (inferenceengineering.co),
// sections "How PagedAttention maps an OS concept onto GPU memory" and "The
// non-contiguous memory layout PagedAttention introduces and its overhead"
// — every attention step follows the block table, and gathering scattered
// pages is the cost to keep small.  Scores are never written to memory (the
// fused-attention property named in the section on block-level eviction).
//
// Matrix-core path (bf16 q; bf16 or E4M3 KV; G = H_q/H_kv <= 16; D 64/128).
//
// Work decomposition.  A segment is one (sequence b, KV head g); its unit of
// work is a 32-token chunk, c_b = ceil(n_b / 32) chunks.  Every workgroup
// reads the lengths and computes the same plan: upw = max(8, ceil(H_kv *
// sum_b c_b / target)) chunks per piece, where target is one round of
// resident workgroups (occupancy x CUs); segment (b, g) is cut into
// np_b = ceil(c_b / upw) pieces of near-equal chunk counts.  Workgroups take
// the pieces largest first (size classes a factor sqrt(2) apart, then
// sequence-major; prefix scans over the sequences find a workgroup's piece),
// so the short pieces fill the slots that free up at the end; workgroups past
// the last piece exit.  So no resident workgroup streams more than about
// upw chunks whatever the length mix, and a batch whose segments all fit one
// round needs no partial results.
// Workgroups have 8 waves when every segment fits one round whole, else 4
// (twice as many workgroups, so one workgroup's start and end overlap
// another's streaming on the same CU).  Inside a piece the waves take chunks
// round-robin and merge through LDS at the end.
//
// Per chunk, per wave:
//   S^T[16 tok][16 heads] = K[16 tok][D] . Q^T[D][16 heads]   two
//     v_mfma_f32_16x16x32_bf16 chains (one per 16-token half); A = K rows
//     straight from the pool, B = the wave's resident Q (heads >= G zero).
//   online softmax in log2 units on the MFMA accumulator layout (lane l holds
//     head l%16, tokens 4*(l/16)+i): the running maximum only moves when a
//     chunk exceeds it by more than 2^8, so the rescale of the accumulators is
//     rare; the sum stays per lane until the end.
//   O[16 heads][D] += P[16 heads][32 tok] . V[32 tok][D] with P split into
//     bf16 hi + lo parts (two MFMAs per tile) so P keeps ~16 bits; P is
//     regrouped across lane groups (permlane32/16 swaps) so that lane group r
//     holds tokens 8r .. 8r+7.
// The pool layout makes every MFMA operand a 16- or 8-byte lane load: the K
// tile is [D/X][bs][X] (16 tokens x 16 bytes contiguous per 16 lanes) and the
// V tile is [D][bs] (8 consecutive tokens of one column per lane), so no LDS
// staging or transposition is needed on the hot loop.
//
// A piece that covers its whole segment writes the final rows; otherwise it
// writes its unnormalised output and (max, sum) per head to the workspace,
// and the segment's last piece to finish combines the pieces in the same
// launch:
//     o = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i,  M = max_i m_i.
// The partials go through agent-scope (cross-XCD coherent) stores and loads
// and the pieces count themselves with one agent-scope compare-and-swap each
// (merge_if_last); a release/acquire fence pair would instead write back and
// invalidate a whole L2 per workgroup, which costs far more.  When the
// caller's length sum shows that no segment would be cut, the launch runs in
// single-piece mode (each workgroup raises upw to the longest segment itself).
//
// Fused step (bf16 pools): the step's new token of each sequence is put into
// the loaded operands of the chunk holding position n - 1 and stored into the
// pool after the chunk loop, which saves the append launch.
//
// The other supported combinations (fp32 q or KV, G > 16, D = 256) take the
// vector path in decode_vector.hip.

#include <hip/hip_runtime.h>

#include <math.h>

#include <mutex>

#include "decode_common.h"
#include "e4m3_encode.h"
#include "internal.h"
#include "tile_ops.h"
#include "wave_scan.h"

namespace pkv {
namespace {

// ---------------------------------------------------------------------------
// matrix-core path
// ---------------------------------------------------------------------------
template <int D, int BS, int KVT>
struct Chunk {
  static constexpr int kKLoads = KVT == PKV_BF16 ? D / 32 : D / 64;  // 16-byte K loads per half
  u32x4 k[2][kKLoads];
  // V operand per output tile: 8 consecutive tokens of one column, as
  // bf16 (4 words) or E4M3 codes (2 words)
  typename std::conditional<KVT == PKV_BF16, u32x4, u32x2>::type v[D / 16];
};

// ids[idx] for a per-lane idx over wave-uniform ids, as a select chain.  Each
// id passes through an empty asm first: otherwise the optimizer turns the
// selects of loads from the local array into one load at a selected index,
// which puts the array in scratch memory (it did at 4 blocks per chunk).
template <int NBCH>
__device__ __forceinline__ int pick(const int (&ids)[NBCH], int idx) {
  int r = ids[0];
  asm("" : "+s"(r));
#pragma unroll
  for (int i = 1; i < NBCH; ++i) {
    int v = ids[i];
    asm("" : "+s"(v));
    r = idx == i ? v : r;
  }
  return r;
}

template <int D, int BS, int KVT>
__device__ __forceinline__ void load_chunk(Chunk<D, BS, KVT>& ch, const char* __restrict__ kpool,
                                           const char* __restrict__ vpool, const int32_t* __restrict__ tab,
                                           int chunk, int last_blk, int NB, int H_kv, int g, int lane) {
  constexpr int S = KvTraits<KVT>::kBytes;
  constexpr int NBCH = BS >= 32 ? 1 : 32 / BS;
  constexpr size_t kTile = (size_t)D * BS * S;
  const int cs = chunk * 32;
  int ids[NBCH];
#pragma unroll
  for (int i = 0; i < NBCH; ++i) ids[i] = block_id(tab, cs / BS + i, last_blk, NB);
  const int m = lane & 15, kg = lane >> 4;
  const size_t gofs = (size_t)g * kTile;
  const size_t bstride = (size_t)H_kv * kTile;
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int tk = 16 * a + m;  // token within the chunk this lane's K row belongs to
    const int id = pick<NBCH>(ids, BS >= 32 ? 0 : tk / BS);
    const char* base = kpool + (size_t)id * bstride + gofs + (size_t)(kg * BS + tk % BS) * 16;
#pragma unroll
    for (int c = 0; c < Chunk<D, BS, KVT>::kKLoads; ++c)
      ch.k[a][c] = __builtin_nontemporal_load((const u32x4*)(base + (size_t)c * 64 * BS));
  }
  // V: lane (n, kg) holds tokens 8kg .. 8kg+7 of column n of each 16-column
  // tile (the B operand of the PV MFMA), one 16- or 8-byte load per tile
  const int n = lane & 15;
  const int tv = 8 * kg;
  const int vid = pick<NBCH>(ids, BS >= 32 ? 0 : tv / BS);
  const char* vbase = vpool + (size_t)vid * bstride + gofs + ((size_t)n * BS + tv % BS) * S;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    const char* p = vbase + (size_t)t * 16 * BS * S;
    if constexpr (KVT == PKV_BF16)
      ch.v[t] = __builtin_nontemporal_load((const u32x4*)p);
    else
      ch.v[t] = __builtin_nontemporal_load((const u32x2*)p);
  }
}

struct WaveState {
  float m;  // running max of head (lane & 15), log2 units, same in the head's 4 lanes
  float l;  // this lane's share of the running sum
};

template <int D, int BS, int KVT>
__device__ __forceinline__ void process_chunk(const Chunk<D, BS, KVT>& ch, const u32x4 (&qop)[D / 32],
                                              f32x4 (&acc)[D / 16], WaveState& st, int chunk, int n,
                                              int hlo, int hhi, float sl, int lane) {
  const int cs = chunk * 32;
  const int kg = lane >> 4;
  // wave-uniform: the chunk holds a token past n or inside the hole [hlo, hhi)
  const bool tail = cs + 32 > n || (cs < hhi && cs + 32 > hlo);
  // ---- S^T = K Q^T for the two 16-token halves
  f32x4 s[2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    s[a] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (KVT == PKV_BF16) {
#pragma unroll
      for (int c = 0; c < D / 32; ++c) s[a] = mfma16x16x32(ch.k[a][c], qop[c], s[a]);
    } else {
#pragma unroll
      for (int u = 0; u < D / 64; ++u) {
        const u32x4 w = ch.k[a][u];
        s[a] = mfma16x16x32(e4m3x8_to_bf16x8(w.x, w.y), qop[2 * u], s[a]);
        s[a] = mfma16x16x32(e4m3x8_to_bf16x8(w.z, w.w), qop[2 * u + 1], s[a]);
      }
    }
  }
  float x[8];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v = s[a][i] * sl;
      if (tail) {
        const int t = cs + 16 * a + 4 * kg + i;
        v = (t < n && (t < hlo || t >= hhi)) ? v : -INFINITY;
      }
      x[4 * a + i] = v;
    }
  // ---- chunk max per head: 8 values in the lane, then the head's 4 lanes
  float cm = x[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) cm = fmaxf(cm, x[j]);
  if constexpr (KVT == PKV_BF16) {
    cm = max_over_groups(cm);
  } else {  // E4M3 at its 3-wave bound: the permlane form spills two registers (2 % slower at bs 32)
    cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
    cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
  }
  const bool need = cm > st.m + kRescaleLog2;
  if (__ballot(need)) {
    const float mu = need ? cm : st.m;
    const float alpha = exp2_fast(st.m - mu);
    st.l *= alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ai = __shfl(alpha, 4 * kg + i, 64);  // alpha of accumulator row 4*kg+i
#pragma unroll
      for (int t = 0; t < D / 16; ++t) acc[t][i] *= ai;
    }
    st.m = mu;
  }
  // ---- P = exp2(x - m): keep the fp32 sum.  bf16 V: P as bf16 hi + lo for two MFMAs; E4M3 V:
  // P and V in fp16 (every E4M3 value is an fp16 value), one MFMA
  float pj[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) pj[j] = exp2_fast(x[j] - st.m);
  if (tail)  // a masked token weighs 0, also while no token has been seen (m = -inf)
#pragma unroll
    for (int j = 0; j < 8; ++j) pj[j] = x[j] == -INFINITY ? 0.f : pj[j];
  float psum = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) psum += pj[j];
  st.l += psum;
  // pairs: words 0,1 = tokens 4kg..4kg+3 of half 0, words 2,3 = the same of half 1
  u32x4 ph, pl;
  if constexpr (KVT == PKV_BF16) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t b0 = __builtin_bit_cast(uint32_t, pj[2 * w]), b1 = __builtin_bit_cast(uint32_t, pj[2 * w + 1]);
      ph[w] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
      pl[w] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, pj[2 * w + 1] - __builtin_bit_cast(float, b1 & 0xFFFF0000u)),
                                    __builtin_bit_cast(uint32_t, pj[2 * w] - __builtin_bit_cast(float, b0 & 0xFFFF0000u)),
                                    0x07060302u);
    }
    pl = tokens_by_eight(pl);
  } else {
#pragma unroll
    for (int w = 0; w < 4; ++w) ph[w] = pack_f16(pj[2 * w], pj[2 * w + 1]);
  }
  ph = tokens_by_eight(ph);
  // ---- V tail mask: k-slot j of lane group kg is token 8kg + j
  u32x4 vmask = u32x4{~0u, ~0u, ~0u, ~0u};
  if (tail) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const int t0 = cs + 8 * kg + 2 * w, t1 = t0 + 1;
      const bool ok0 = t0 < n && (t0 < hlo || t0 >= hhi), ok1 = t1 < n && (t1 < hlo || t1 >= hhi);
      vmask[w] = (ok0 ? 0x0000FFFFu : 0u) | (ok1 ? 0xFFFF0000u : 0u);
    }
  }
  // ---- O += P V
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    if constexpr (KVT == PKV_BF16) {
      u32x4 vop = ch.v[t];
      if (tail) vop &= vmask;
      acc[t] = mfma16x16x32(ph, vop, acc[t]);
      acc[t] = mfma16x16x32(pl, vop, acc[t]);
    } else {
      u32x4 vop = e4m3x8_to_f16x8(ch.v[t][0], ch.v[t][1]);
      if (tail) vop &= vmask;
      acc[t] = mfma16x16x32_f16(ph, vop, acc[t]);
    }
  }
}

// The fused step's new token of one (sequence, KV head) as E4M3 codes, K then V (D <= 128), in LDS.
__shared__ __align__(16) uint8_t sh_newtok[2 * 128];

// ---------------------------------------------------------------------------
// fused step (append + decode): the step's new token of (b, g) at position n - 1
// ---------------------------------------------------------------------------
// Put the new token straight into the loaded operands of the chunk holding
// position n - 1 (tk = its offset in the chunk, wave-uniform), as the pool will
// hold it: a bf16 pool stores the row's bits as they are, an E4M3 pool the codes
// of x / scale (the append's encoding, taken once per piece into LDS before the
// chunk loop: codes[0, D) for K, codes[D, 2 D) for V), so the decode sees the
// appended token while the pool store waits until after the chunk loop.
template <int D, int BS, int KVT>
__device__ __forceinline__ void inject_new_token(Chunk<D, BS, KVT>& ch, const DecodeArgs& a, int b, int g, int tk,
                                                 const uint8_t* codes, int lane) {
  const uint16_t* nk = (const uint16_t*)a.new_k + ((size_t)b * a.H_kv + g) * D;
  const uint16_t* nv = (const uint16_t*)a.new_v + ((size_t)b * a.H_kv + g) * D;
  const int m = lane & 15, kg = lane >> 4;
  if (m == (tk & 15)) {  // K: lane m of half tk / 16 holds the token's row, dim groups kg + 4c
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      if (half != (tk >> 4)) continue;
#pragma unroll
      for (int c = 0; c < Chunk<D, BS, KVT>::kKLoads; ++c) {
        if constexpr (KVT == PKV_BF16) {
          ch.k[half][c] = *(const u32x4*)(nk + (kg + 4 * c) * 8);
        } else {  // codes of dims 16 (kg + 4 c) .. + 15
          ch.k[half][c] = *(const u32x4*)(codes + 16 * (kg + 4 * c));
        }
      }
    }
  }
  if (kg == (tk >> 3)) {  // V: element tk % 8 of lane (m, kg)'s 8 tokens of column 16 t + m
    const int j = tk & 7;
#pragma unroll
    for (int t = 0; t < D / 16; ++t) {
      if constexpr (KVT == PKV_BF16) {
        const uint32_t x = nv[16 * t + m];
        const int sh = 16 * (j & 1);
#pragma unroll
        for (int wd = 0; wd < 4; ++wd)
          if (wd == j / 2) ch.v[t][wd] = (ch.v[t][wd] & ~(0xFFFFu << sh)) | (x << sh);
      } else {
        const int sh = 8 * (j & 3);
        const uint32_t code = codes[D + 16 * t + m];
#pragma unroll
        for (int wd = 0; wd < 2; ++wd)
          if (wd == j / 4) ch.v[t][wd] = (ch.v[t][wd] & ~(0xFFu << sh)) | (code << sh);
      }
    }
  }
}

// The pool store of the new token's K and V rows of head g (one wave, after
// the chunk loop), the same bytes pkv_kv_append writes into the pool.
template <int D, int BS, int KVT>
__device__ __forceinline__ void write_new_token(const DecodeArgs& a, int b, int g, long long slot,
                                                const uint8_t* codes, int lane) {
  const uint16_t* nk = (const uint16_t*)a.new_k + ((size_t)b * a.H_kv + g) * D;
  const uint16_t* nv = (const uint16_t*)a.new_v + ((size_t)b * a.H_kv + g) * D;
  const int off = (int)(slot % BS);
  if constexpr (KVT == PKV_BF16) {
    const size_t tile = ((size_t)(slot / BS) * a.H_kv + g) * (size_t)D * BS;  // bf16 elements
    uint16_t* kp = (uint16_t*)a.k_pool + tile;
    uint16_t* vp = (uint16_t*)a.v_pool + tile;
    if (lane < D / 8)  // K [D/8][BS][8]: one 16-byte dim group per lane
      *(u32x4*)(kp + ((size_t)lane * BS + off) * 8) = *(const u32x4*)(nk + lane * 8);
    for (int d = lane; d < D; d += 64) vp[(size_t)d * BS + off] = nv[d];  // V [D][BS]
  } else {
    const size_t tile = ((size_t)(slot / BS) * a.H_kv + g) * (size_t)D * BS;  // bytes
    uint8_t* kp = (uint8_t*)a.k_pool + tile;
    uint8_t* vp = (uint8_t*)a.v_pool + tile;
    if (lane < D / 16)  // K [D/16][BS][16]: one 16-code dim group per lane
      *(u32x4*)(kp + ((size_t)lane * BS + off) * 16) = *(const u32x4*)(codes + 16 * lane);
    for (int d = lane; d < D; d += 64) vp[(size_t)d * BS + off] = codes[D + d];  // V [D][BS]
  }
}

// ---------------------------------------------------------------------------
// matrix-core path: one piece per workgroup, pieces planned from the lengths
//
// The batch's work is c_b = ceil(n_b / 32) chunks per (sequence b, KV head g)
// segment.  Every workgroup derives the same plan from the lengths: with
// total = H_kv * sum_b c_b units and T target pieces (the workgroups the GPU
// holds at once), upw = ceil(total / T), and each segment of sequence b is cut
// into np_b = ceil(c_b / upw) balanced pieces, numbered sequence-major, then
// KV head, then piece (the workspace row of a piece's partials).  Workgroup i
// takes the i-th piece in size-class order (largest class first, then that
// numbering; see plan_piece).  A uniform batch thus runs as exactly one round
// of equal pieces (no second-round bubble); a batch of mixed lengths gets many
// segment-aligned pieces, at most upw chunks each, which the hardware
// dispatcher balances.  Each workgroup runs a single piece,
// which keeps register use (and so occupancy) at its single-piece minimum.
// The workgroup's NW (4 or 8) waves take the piece's chunks round-robin and
// merge through LDS; a piece that is a whole segment writes its final rows,
// the others write partials that the segment's last piece combines.
// ---------------------------------------------------------------------------
constexpr int kMinUnits = 8;
constexpr int kLensInRegs = 16;  // lengths a lane keeps in registers (B <= 1024 in one pass)

__device__ __forceinline__ int chunks_of(int n, int cap) {
  n = n < 0 ? 0 : (n > cap ? cap : n);
  return (n + 31) / 32;
}

struct PiecePlan {
  int b, g, n, lo, hi, np;  // piece [lo, hi) of segment (b, g); np pieces in the segment; n = its length
  int id;                   // the piece's number in sequence-major order (its workspace row)
  int first;                // the number of the segment's first piece
};

constexpr int kSizeClasses = 8;  // piece-size classes, a factor sqrt(2) apart

// ceil(c / u) for c >= 0 and a divisor u >= kMinUnits that is the same in every lane: a float
// estimate of the quotient, corrected once each way, which is exact while c < 2^24 (the estimate
// is then within 0.4 of c / u); larger counts take the integer division.
__device__ __forceinline__ int ceil_div_units(int c, int u) {
  if (c >= (1 << 24)) return (c + u - 1) / u;
  int q = (int)((float)c * __builtin_amdgcn_rcpf((float)u));
  int r = c - q * u;
  if (r < 0) {
    q -= 1;
    r += u;
  }
  if (r >= u) {
    q += 1;
    r -= u;
  }
  return q + (r > 0);
}

// Size class of a segment cut into np pieces from c chunks: floor(2 log2(upw * np / c)), clamped
// to [0, kSizeClasses - 1], i.e. the pieces hold about upw / sqrt(2)^k chunks in class k; class 0
// holds the largest.  v_log_f32 gives the same bits for the same inputs in every wave, so every
// pass of every workgroup puts a segment in the same class.
__device__ __forceinline__ int size_class(int c, int np, int upw) {
  const float k = 2.f * (__builtin_amdgcn_logf((float)upw * (float)np) - __builtin_amdgcn_logf((float)c));
  const int ki = (int)k;
  return ki < 0 ? 0 : (ki > kSizeClasses - 1 ? kSizeClasses - 1 : ki);
}

// Chunks per piece (upw) of the plan, from the lengths; every wave that calls it gets the same
// value.  nl receives the clamped lengths of sequences lane, lane + 64, ... (the first
// kLensInRegs * 64 sequences; len_at reads the rest from memory again).
__device__ int plan_upw(const DecodeArgs& a, int target, int lane, int (&nl)[kLensInRegs]) {
  const int B = a.B, cap = a.len_cap;
  int part = 0, cmax = 0;
#pragma unroll
  for (int k = 0; k < kLensInRegs; ++k) {
    const int b0 = lane + 64 * k;
    nl[k] = b0 < B ? seq_len(a.context_lens, b0, cap) : 0;
    const int cb = (nl[k] + 31) / 32;
    part += cb;
    cmax = max(cmax, cb);
  }
  for (int b0 = lane + 64 * kLensInRegs; b0 < B; b0 += 64) {
    const int cb = chunks_of(a.context_lens[b0], cap);
    part += cb;
    cmax = max(cmax, cb);
  }
  const int total = uniform(wave_sum(part)) * a.H_kv;
  int upw = (total + target - 1) / target;
  upw = upw < kMinUnits ? kMinUnits : upw;
  if (a.single_piece) {  // every segment whole, whatever the host's estimate was
    const int m = uniform(wave_max(cmax));
    upw = upw < m ? m : upw;
  }
  return upw;
}

// clamped length of sequence lane + 64 k (0 past the batch)
__device__ __forceinline__ int len_at(const DecodeArgs& a, const int (&nl)[kLensInRegs], int k, int lane) {
  int n = 0;
  if (k < kLensInRegs) {
#pragma unroll
    for (int kk = 0; kk < kLensInRegs; ++kk) n = kk == k ? nl[kk] : n;
  } else {
    const int b0 = lane + 64 * k;
    n = b0 < a.B ? seq_len(a.context_lens, b0, a.len_cap) : 0;
  }
  return n;
}

// The piece that workgroup `item` runs (one wave computes it; pp.b = -1 if none).
//
// Pieces are numbered sequence-major (segment (b, g) owns np_b consecutive numbers) and that
// number is the piece's workspace row, which the merge finds again from the lengths alone.  The
// workgroups take them in another order: size class by size class, largest first, and
// sequence-major inside a class.  The dispatcher starts workgroups in grid order, so long pieces
// start in the first round and the short ones fill the slots that free up at the end (a
// longest-first list schedule, to within a factor sqrt(2) of piece size).
__device__ void plan_piece(const DecodeArgs& a, int target, int item, int lane, PiecePlan& pp) {
  const int B = a.B, H_kv = a.H_kv;
  int nl[kLensInRegs];
  const int upw = plan_upw(a, target, lane, nl);
  pp.b = -1;
  // size class of every sequence's pieces; a batch in one class needs no class counts
  int ccnt[kSizeClasses];
#pragma unroll
  for (int kk = 0; kk < kSizeClasses; ++kk) ccnt[kk] = 0;
  int cls0 = -1;
  bool mixed = false;
  for (int k = 0; k * 64 < B; ++k) {
    const int n = len_at(a, nl, k, lane);
    const int cb = (n + 31) / 32, npb = ceil_div_units(cb, upw);
    const int cls = npb > 0 ? size_class(cb, npb, upw) : -1;
    if (k == 0) cls0 = uniform(cls);  // sequence 0's class (-1: empty)
    mixed = mixed || (cls >= 0 && cls != cls0);
#pragma unroll
    for (int kk = 0; kk < kSizeClasses; ++kk) ccnt[kk] += kk == cls ? npb * H_kv : 0;
  }
  mixed = __ballot(mixed) != 0ull;
  // the class holding `item`, and its rank r inside that class (-1: every class)
  int cls_item = -1, r = item;
  if (mixed) {
#pragma unroll
    for (int kk = 0; kk < kSizeClasses; ++kk) {
      const int tot = uniform(wave_sum(ccnt[kk]));
      if (cls_item < 0) {
        if (r < tot)
          cls_item = kk;
        else
          r -= tot;
      }
    }
    if (cls_item < 0) return;  // past the last piece
  }
  // locate rank r among the class's pieces (sequence-major), with the sequence-major number
  int base = 0, cbase = 0;
  for (int k = 0; k * 64 < B && pp.b < 0; ++k) {
    const int n = len_at(a, nl, k, lane);
    const int cb = (n + 31) / 32, npb = ceil_div_units(cb, upw);
    const int all = npb * H_kv;
    const int cnt = cls_item < 0 || (npb > 0 && size_class(cb, npb, upw) == cls_item) ? all : 0;
    const int incl = wave_incl_scan(cnt);
    const int call = wave_incl_scan(all);
    const bool hit = cnt > 0 && base + incl - cnt <= r && r < base + incl;
    const unsigned long long m = __ballot(hit);
    if (m) {
      const int src = __ffsll((long long)m) - 1;
      const int rr = r - lane_value(base + incl - cnt, src);  // = g * np + j inside the sequence
      const int np = lane_value(npb, src), cbb = lane_value(cb, src);
      const int j = rr % np;
      pp.b = 64 * k + src;
      pp.g = rr / np;
      pp.np = np;
      pp.n = lane_value(n, src);
      pp.id = lane_value(cbase + call - all, src) + rr;
      pp.first = pp.id - j;
      pp.lo = (int)((long long)j * cbb / np);
      pp.hi = (int)((long long)(j + 1) * cbb / np);
    }
    base += lane_value(incl, 63);
    cbase += lane_value(call, 63);
  }
  pp.b = uniform(pp.b);
}

// process one chunk; in the fused step the new token enters the operands of
// its chunk just before they are used
template <int D, int BS, int KVT, bool APPEND>
__device__ __forceinline__ void proc_chunk(Chunk<D, BS, KVT>& X, const DecodeArgs& a, const u32x4 (&qop)[D / 32],
                                           f32x4 (&acc)[D / 16], WaveState& st, int c, int n, int hlo, int hhi,
                                           float sl, int inject_chunk, int b, int g, int lane) {
  if constexpr (APPEND)
    if (c == inject_chunk) inject_new_token(X, a, b, g, n - 1 - 32 * c, sh_newtok, lane);
  process_chunk(X, qop, acc, st, c, n, hlo, hhi, sl, lane);
}

// The wave's share of one piece: chunks first, first + NW, ... below c_end of
// segment (b, g), with the next chunk's loads in flight while one is computed.
// resident Q operand of KV head g of sequence b: lane holds head (lane & 15), 8 head-dim values
// per MFMA (heads >= G zero)
template <int D, int KVT>
__device__ __forceinline__ void load_q(u32x4 (&qop)[D / 32], const DecodeArgs& a, int b, int g, int lane) {
  const int h = lane & 15, kg = lane >> 4;
  const uint16_t* qrow = (const uint16_t*)a.q + ((size_t)b * a.H_q + g * a.G + h) * D;
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (h < a.G) v = *(const u32x4*)(qrow + qk_dofs<KVT>(c, kg));
    qop[c] = v;
  }
}

// The wave's share of one piece: chunks first, first + NW, ... below c_end of segment (b, g),
// with the next chunk's loads in flight while one is computed.  With `pre`, qop and A already hold
// the Q operand and chunk `first` (loaded before the plan was known).
template <int D, int BS, int KVT, int NW, bool APPEND>
__device__ __forceinline__ void run_piece(const DecodeArgs& a, int b, int g, int n, int hlo, int hhi, int first,
                                          int c_end, int inject_chunk, f32x4 (&acc)[D / 16], WaveState& st,
                                          Chunk<D, BS, KVT>& A, u32x4 (&qop)[D / 32], bool pre, int lane) {
  const int last_blk = (n + BS - 1) / BS - 1;
  const int32_t* tab = a.block_tables + (size_t)b * a.max_blocks;
  const char* kpool = (const char*)a.k_pool;
  const char* vpool = (const char*)a.v_pool;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  st = WaveState{-INFINITY, 0.f};
  const int cnt = first < c_end ? (c_end - first + NW - 1) / NW : 0;
  if (cnt == 0) return;
  if (!pre) load_q<D, KVT>(qop, a, b, g, lane);
  float sl = a.scale_log2;
  if constexpr (KVT == PKV_FP8_E4M3) sl *= a.k_scale[g];
  Chunk<D, BS, KVT> Bf;
  int c = first;
  if (!pre) load_chunk(A, kpool, vpool, tab, c, last_blk, a.NB, a.H_kv, g, lane);
  int k = 0;
  for (; k + 2 < cnt; k += 2) {
    load_chunk(Bf, kpool, vpool, tab, c + NW, last_blk, a.NB, a.H_kv, g, lane);
    proc_chunk<D, BS, KVT, APPEND>(A, a, qop, acc, st, c, n, hlo, hhi, sl, inject_chunk, b, g, lane);
    load_chunk(A, kpool, vpool, tab, c + 2 * NW, last_blk, a.NB, a.H_kv, g, lane);
    proc_chunk<D, BS, KVT, APPEND>(Bf, a, qop, acc, st, c + NW, n, hlo, hhi, sl, inject_chunk, b, g, lane);
    c += 2 * NW;
  }
  if (k + 1 < cnt) {
    load_chunk(Bf, kpool, vpool, tab, c + NW, last_blk, a.NB, a.H_kv, g, lane);
    proc_chunk<D, BS, KVT, APPEND>(A, a, qop, acc, st, c, n, hlo, hhi, sl, inject_chunk, b, g, lane);
    proc_chunk<D, BS, KVT, APPEND>(Bf, a, qop, acc, st, c + NW, n, hlo, hhi, sl, inject_chunk, b, g, lane);
  } else {
    proc_chunk<D, BS, KVT, APPEND>(A, a, qop, acc, st, c, n, hlo, hhi, sl, inject_chunk, b, g, lane);
  }
}

// Merge of a cut segment inside the piece kernel, by the piece that finishes last.  Every piece
// stores its partials with agent-scope stores (they reach the level the XCDs share), the
// workgroup's barrier waits for them, and one thread then counts the piece in the segment's
// arrival word with an agent-scope compare-and-swap: the word holds (call token, pieces arrived),
// and a word carrying another token counts as 0, so neither a previous call's word nor
// uninitialised memory is taken for this call's.  The piece that brings the count to np clears the
// word and combines the np partials (agent-scope loads) into the output rows:
//     o = sum_i 2^(m_i - M) o_i / sum_i 2^(m_i - M) l_i,  M = max_i m_i.
// No piece waits for another, so nothing can hang on a piece that runs late.
constexpr int kMergeBatch = 8;

template <int NT>
__device__ void merge_if_last(const DecodeArgs& a, int b, int g, int np, int first, size_t orow, int tid) {
  __shared__ int sh_last;
  __syncthreads();  // every thread's partial stores have completed
  if (tid == 0) {
    unsigned long long* ctr = a.ws_ctr + ((size_t)b * a.H_kv + g);
    const unsigned long long tag = (unsigned long long)a.call_token << 32;
    // first guess: this piece is the last one (one round trip when it is, the case whose latency
    // ends the segment); a failed exchange returns the word as it is
    unsigned long long cur = tag | (unsigned long long)(np - 1);
    unsigned long long arrived;
    do {
      arrived = ((cur >> 32) == a.call_token ? (cur & 0xFFFFFFFFull) : 0ull) + 1ull;
    } while (!__hip_atomic_compare_exchange_strong(ctr, &cur, tag | arrived, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT));
    const bool last = arrived == (unsigned long long)np;
    if (last) __hip_atomic_store(ctr, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);  // clean for later calls
    sh_last = last;
  }
  __syncthreads();
  if (!sh_last) return;
  const int G = a.G, D = a.D;
  for (int e = tid; e < G * D; e += NT) {
    const int hl = e / D, col = e % D;
    float M = -INFINITY, L = 0.f, O = 0.f;
    for (int p = 0; p < np; p += kMergeBatch) {
      float mp[kMergeBatch], lp[kMergeBatch], op[kMergeBatch];
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) {  // past the last piece: reload the last, weigh it 0
        const size_t r = (size_t)(first + min(p + i, np - 1)) * 16 + hl;
        mp[i] = __hip_atomic_load(&a.ws_ml[2 * r], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lp[i] = __hip_atomic_load(&a.ws_ml[2 * r + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        op[i] = __hip_atomic_load(&a.ws_o[r * D + col], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int i = 0; i < kMergeBatch; ++i) {
        if (p + i >= np || mp[i] == -INFINITY) continue;  // no piece, or one that attended nothing
        const float mn = fmaxf(M, mp[i]);
        const float so = M == -INFINITY ? 0.f : exp2_fast(M - mn);
        const float sn = exp2_fast(mp[i] - mn);
        L = L * so + lp[i] * sn;
        O = O * so + op[i] * sn;
        M = mn;
      }
    }
    a.out[orow + e] = L > 0.f ? O / L : 0.f;  // nothing attended: zero row
  }
}

template <int D, int BS, int KVT, int NW, bool APPEND>
__global__ __launch_bounds__(64 * NW, KVT == PKV_FP8_E4M3 ? 3 : 2) void decode_piece_kernel(DecodeArgs a,
                                                                                          int target) {
  constexpr int NT = 64 * NW;
  __shared__ float sh_acc[NW][16][D];
  __shared__ float sh_m[NW][16];
  __shared__ float sh_l[NW][16];
  const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
  const int item = blockIdx.x;
  const int G = a.G, cap = a.len_cap;
  // a sequence with no tokens: zero rows, written by workgroup b.
  // Only float stores may come before the chunk loop: the compiler keeps the
  // block-table and length reads on the scalar unit only while it can prove
  // that no earlier store of the kernel overwrites them, and an int32 store
  // (same type as the tables) would turn them into vector loads with a full
  // wait for memory on every chunk.
  if (item < a.B && uniform(seq_len(a.context_lens, item, cap)) == 0)
    for (int e = tid; e < a.H_q * D; e += NT) a.out[(size_t)item * a.H_q * D + e] = 0.f;
  // When the caller's length sum says every length equals len_cap (single-piece mode, one size
  // class, no empty sequence), workgroup `item` runs segment (item / H_kv, item % H_kv) whole:
  // every wave loads that guess's Q operand and its first chunk before the plan is known, so the
  // loads overlap the plan's round trip; a plan that disagrees (a wrong sum) loads again.  The guess's block indices are clamped
  // to the table row (the plan's clamp is the sequence's last block); the blocks the two clamps
  // can differ on hold only positions past the sequence's end, which the chunk's masks drop.
  Chunk<D, BS, KVT> A;
  u32x4 qop[D / 32];
  const int guess_b = item / a.H_kv, guess_g = item % a.H_kv;
  const bool guess = a.speculate && guess_b < a.B;
  if (guess) {
    load_q<D, KVT>(qop, a, guess_b, guess_g, lane);
    load_chunk(A, (const char*)a.k_pool, (const char*)a.v_pool, a.block_tables + (size_t)guess_b * a.max_blocks, w,
               a.max_blocks - 1, a.NB, a.H_kv, guess_g, lane);
  }
  // wave 0 plans; the other waves wait at the barrier rather than repeat its scalar work
  __shared__ int sh_plan[8];
  if (w == 0) {
    PiecePlan pp;
    plan_piece(a, target, item, lane, pp);
    if (lane == 0) {
      sh_plan[0] = pp.b;
      sh_plan[1] = pp.g;
      sh_plan[2] = pp.np;
      sh_plan[3] = pp.lo;
      sh_plan[4] = pp.hi;
      sh_plan[5] = pp.n;
      sh_plan[6] = pp.id;
      sh_plan[7] = pp.first;
    }
  }
  __syncthreads();
  const int b = uniform(sh_plan[0]), g = uniform(sh_plan[1]);
  // no piece for this workgroup (a plan naming a segment outside the batch runs nothing either)
  if (b < 0 || b >= a.B || (unsigned)g >= (unsigned)a.H_kv) return;
  const int np = uniform(sh_plan[2]), lo = uniform(sh_plan[3]), hi = uniform(sh_plan[4]);
  const int n = uniform(sh_plan[5]), pid = uniform(sh_plan[6]), first_pid = uniform(sh_plan[7]);
  int hlo, hhi;
  seq_hole(a, b, hlo, hhi);
  hlo = uniform(hlo);
  hhi = uniform(hhi);
  // fused step: the piece holding position n - 1 takes the new token from the
  // step's rows when its slot is that position's slot (else the pool is read as is)
  int inject_chunk = -1;
  bool writer = false;  // this piece stores the new token into the pool after its loop
  long long new_slot = -1;
  if constexpr (APPEND) {
    new_slot = a.new_slots[b];
    const int last = n - 1, uc = last / 32;
    writer = n > 0 && lo <= uc && uc < hi && new_slot >= 0 && new_slot < (long long)a.NB * BS;
    if (writer) {
      const int32_t* tab = a.block_tables + (size_t)b * a.max_blocks;
      const long long expect = (long long)tab[last / BS] * BS + last % BS;
      if (expect == new_slot) inject_chunk = uc;
    }
    inject_chunk = uniform(inject_chunk);
    if constexpr (KVT == PKV_FP8_E4M3) {
      if (writer) {  // the new token's codes, once, before any wave's chunk loop takes them
        const uint16_t* nk = (const uint16_t*)a.new_k + ((size_t)b * a.H_kv + g) * D;
        const uint16_t* nv = (const uint16_t*)a.new_v + ((size_t)b * a.H_kv + g) * D;
        const float ks = a.k_scale[g], vsc = a.v_scale[g];
        for (int e = tid; e < 2 * D; e += NT)
          sh_newtok[e] = (uint8_t)(e < D ? bf16_to_e4m3(nk[e], ks) : bf16_to_e4m3(nv[e - D], vsc));
        __syncthreads();
      }
    }
  }
  f32x4 acc[D / 16];
  WaveState st;
  const bool pre = guess && b == guess_b && g == guess_g && lo == 0;
  run_piece<D, BS, KVT, NW, APPEND>(a, b, g, n, hlo, hhi, lo + w, hi, inject_chunk, acc, st, A, qop, pre, lane);
  // ---- merge the NW waves' shares through LDS
  const int kg = lane >> 4;
  float lt = st.l;
  lt += __shfl_xor(lt, 16, 64);
  lt += __shfl_xor(lt, 32, 64);
  if (lane < 16) {
    sh_m[w][lane] = st.m;
    sh_l[w][lane] = lt;
  }
#pragma unroll
  for (int t = 0; t < D / 16; ++t)
#pragma unroll
    for (int i = 0; i < 4; ++i) sh_acc[w][4 * kg + i][16 * t + (lane & 15)] = acc[t][i];
  __syncthreads();
  const float vs = KVT == PKV_FP8_E4M3 ? a.v_scale[g] : 1.f;
  const size_t orow = ((size_t)b * a.H_q + g * G) * D;
  const size_t prow = (size_t)pid * 16;  // workspace row: the sequence-major piece number
  for (int e = tid; e < G * D; e += NT) {
    const int hh = e / D, col = e % D;
    float M = sh_m[0][hh];
#pragma unroll
    for (int i = 1; i < NW; ++i) M = fmaxf(M, sh_m[i][hh]);
    float L = 0.f, O = 0.f;
#pragma unroll
    for (int i = 0; i < NW; ++i) {  // a wave that attended nothing (m = -inf) weighs 0
      const float wt = sh_m[i][hh] == -INFINITY ? 0.f : exp2_fast(sh_m[i][hh] - M);
      L += wt * sh_l[i][hh];
      O += wt * sh_acc[i][hh][col];
    }
    O *= vs;
    if (np == 1) {
      a.out[orow + e] = L > 0.f ? O / L : 0.f;  // nothing attended: zero row
    } else {  // partials, coherent across the XCDs' caches (agent scope)
      __hip_atomic_store(&a.ws_o[(prow + hh) * D + col], O, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (col == 0) {
        __hip_atomic_store(&a.ws_ml[2 * (prow + hh)], M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        __hip_atomic_store(&a.ws_ml[2 * (prow + hh) + 1], L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  if (np > 1) merge_if_last<NT>(a, b, g, np, first_pid, orow, tid);
  if constexpr (APPEND)
    if (writer && w == 0) write_new_token<D, BS, KVT>(a, b, g, new_slot, sh_newtok, lane);
}

// workgroups of decode_piece_kernel<D, BS, KVT, NW, APPEND> one CU holds at once
template <int D, int BS, int KVT, int NW, bool APPEND>
int piece_groups_per_cu() {
  static const int per_cu = [] {
    int nb = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, decode_piece_kernel<D, BS, KVT, NW, APPEND>, 64 * NW, 0) !=
            hipSuccess ||
        nb <= 0)
      nb = 1;
    return nb > kMaxGroupsPerCU ? kMaxGroupsPerCU : nb;
  }();
  return per_cu;
}

template <int D, int BS, int KVT, bool APPEND>
hipError_t launch_mfma_a(const DecodeArgs& a, hipStream_t s) {
  // target pieces = one round of resident workgroups; the plan never makes more
  // than target + B * H_kv pieces, which sizes the grid (the rest exit at once).
  // 8-wave workgroups when every (sequence, KV head) segment fits one round
  // whole: a uniform batch then needs no partials at all.  With bf16 pools
  // also up to two rounds of segments: measured on seeded batches of 48-64
  // sequences with uniform lengths up to 4096 or 8192 tokens (384-512
  // segments), 8 waves were 1-4 % faster in 7 of 8 batches; at 2048 segments
  // (256 sequences of mixed lengths) they were 2-5 % slower.  Otherwise 4-wave
  // workgroups, twice as many, so that piece boundaries of one workgroup
  // overlap another's streaming on the same CU (E4M3 keeps 3 of them per CU).
  const long long segments = (long long)a.B * a.H_kv;
  const int target8 = piece_groups_per_cu<D, BS, KVT, 8, APPEND>() * a.num_cus;
  const bool wide = segments <= target8 || (KVT == PKV_BF16 && segments <= 2LL * target8);
  const int target = wide ? target8 : piece_groups_per_cu<D, BS, KVT, 4, APPEND>() * a.num_cus;
  long long grid = (long long)target + segments;
  // Single-piece mode when the caller's length sum shows that the plan would not cut any
  // segment: ceil(sum / 32) is at most the sum of per-sequence chunk counts, so upw_lo is at
  // most the plan's upw; if even upw_lo covers the longest segment the plan is one piece per
  // segment and no piece writes partials.  The kernel then raises upw to its own
  // longest segment, so a wrong sum only changes the balance of the work and the order of the
  // reduction (the result stays within rounding, not always bit for bit).
  DecodeArgs b = a;
  b.single_piece = 0;
  b.speculate = 0;
  if (a.sum_len_hint >= 0) {
    // cmax <= max(kMinUnits, ceil(csum * H_kv / target)), written without a product of csum
    const long long cmax = ((long long)a.len_cap + 31) / 32;
    const long long csum = a.sum_len_hint / 32 + (a.sum_len_hint % 32 != 0);  // at most B * len_cap / 32 + 1
    b.single_piece = cmax <= kMinUnits || csum > (cmax - 1) * target / a.H_kv;
    // every length at len_cap: one size class and no empty sequence, so workgroup i's segment is
    // (i / H_kv, i % H_kv), which the kernel checks against its plan before using the early loads
    b.speculate = b.single_piece && a.len_cap > 0 && a.sum_len_hint == (long long)a.B * a.len_cap;
    // one piece per segment at most: workgroups past B * H_kv would only plan and exit, and on a
    // batch of one round they are dispatched at the end, as the last segments finish
    if (b.single_piece) grid = segments;
  }
  if (wide)
    hipLaunchKernelGGL((decode_piece_kernel<D, BS, KVT, 8, APPEND>), dim3((unsigned)grid), dim3(512), 0, s, b, target);
  else
    hipLaunchKernelGGL((decode_piece_kernel<D, BS, KVT, 4, APPEND>), dim3((unsigned)grid), dim3(256), 0, s, b, target);
  return hipGetLastError();  // cut segments are merged inside the launch
}

template <int D, int BS, int KVT>
hipError_t launch_mfma_t(const DecodeArgs& a, hipStream_t s) {
  if (a.new_k) return launch_mfma_a<D, BS, KVT, true>(a, s);
  return launch_mfma_a<D, BS, KVT, false>(a, s);
}

template <int D, int KVT>
hipError_t launch_mfma_bs(const DecodeArgs& a, hipStream_t s) {
  switch (a.bs) {
    case 8: return launch_mfma_t<D, 8, KVT>(a, s);
    case 16: return launch_mfma_t<D, 16, KVT>(a, s);
    case 32: return launch_mfma_t<D, 32, KVT>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

// Partials of pkv_paged_attn_decode_noalloc (the same layout a caller's workspace holds).  Each
// device that loads the library holds its own copy until the process ends; every call on a device
// shares it, so calls that overlap on one device race.  Nothing in it has to start at zero: a call
// writes every partial it reads.  Host code never passes the array's name to a kernel (on the host
// it is only a stand-in); it uses the device address static_scratch looked up.
static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

hipError_t static_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {  // once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

bool decode_fast_path_supported(int q_dtype, int kv_dtype, int G, int D, int bs) {
  return q_dtype == PKV_BF16 && (kv_dtype == PKV_BF16 || kv_dtype == PKV_FP8_E4M3) && G >= 1 && G <= 16 &&
         (D == 64 || D == 128) && (bs == 8 || bs == 16 || bs == 32);
}

hipError_t launch_decode_mfma(const DecodeArgs& a, hipStream_t s) {
  if (a.kv_dtype == PKV_BF16) {
    if (a.D == 64) return launch_mfma_bs<64, PKV_BF16>(a, s);
    if (a.D == 128) return launch_mfma_bs<128, PKV_BF16>(a, s);
  } else {
    if (a.D == 64) return launch_mfma_bs<64, PKV_FP8_E4M3>(a, s);
    if (a.D == 128) return launch_mfma_bs<128, PKV_FP8_E4M3>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pkv
