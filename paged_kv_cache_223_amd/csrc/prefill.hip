// Paged prefill (chunked multi-query attention) for gfx950 (CDNA4).
//
// Method: "Paged Attention and KV Cache Fragmentation" (inferenceengineering.co),
// section "How PagedAttention maps an OS concept onto GPU memory": a sequence
// takes blocks as it grows; a prompt, or each chunk of it, is appended into
// them and then attends, causally, over everything before it through the
// same block table the decode walks.  Query i of the C_b new tokens of
// sequence b sits at position p = n_b - C_b + i and attends positions 0..p.
//
// Tiles.  An MFMA column tile is 16 (query token, head) pairs of one KV head g:
// 16 / G consecutive query tokens times the G query heads that share g.  The
// QK^T and PV steps are the decode's (S^T = K Q^T, P split into bf16 hi + lo,
// P regrouped across lane groups, O += P V); only the mask differs: column
// (token at p, head) keeps key t iff t <= p.
//
// Workgroups.  NW waves with R column tiles each cover NW * R * 16 / G
// consecutive query tokens of one (sequence, KV head); every K and V operand
// a wave reads from LDS serves its R tiles.  They share every 32-token K/V
// chunk through LDS: the workgroup copies the chunk's pool tiles (bytes as in
// the pool) into one LDS buffer while the waves compute the previous chunk from
// the other, with the chunk after that already loading into registers, so
// each chunk crosses the L2 once per workgroup, not once per wave.  Work
// items are dealt to the 8 XCDs so that the workgroups of one (sequence, KV
// head) share one XCD's L2, and the latest (longest) tiles of a sequence are
// dispatched first.

#include <hip/hip_runtime.h>

#include <math.h>

#include <type_traits>

#include "internal.h"
#include "tile_ops.h"

namespace pkv {
namespace {

constexpr int kStages = 2;  // the chunk being computed and the next one, written at the iteration's start

template <int D, int BS, int KVT>
struct Stage {
  static constexpr int S = KvTraits<KVT>::kBytes;
  static constexpr int NBCH = BS >= 32 ? 1 : 32 / BS;  // blocks of one 32-token chunk
  static constexpr int kTile = D * BS * S;             // one block's tile of one head (K or V)
  static constexpr int kBytes = 2 * NBCH * kTile;      // the chunk in LDS: K tiles, then V tiles
  static constexpr int kUnits = kBytes / 16;
};

// Copy one chunk's tiles (global -> registers); the workgroup's threads take
// 16-byte units round-robin.  Blocks past the sequence's last block read the
// last block again (masked later), so every access stays inside the pool.
template <int D, int BS, int KVT, int NT>
struct Stager {
  using St = Stage<D, BS, KVT>;
  static constexpr int kPer = (St::kUnits + NT - 1) / NT;
  u32x4 r[kPer];

  __device__ __forceinline__ void load(const char* __restrict__ kpool, const char* __restrict__ vpool,
                                       const int32_t* __restrict__ tab, int chunk, int last_blk, int NB,
                                       int H_kv, int g, int tid) {
    constexpr int tileU = St::kTile / 16;
    const size_t bstride = (size_t)H_kv * St::kTile;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int u = tid + k * NT;
      if (St::kUnits % NT == 0 || u < St::kUnits) {
        const int part = u / (St::NBCH * tileU);  // 0 = K, 1 = V
        const int w = u % (St::NBCH * tileU);
        const int i = w / tileU;
        const int id = block_id(tab, chunk * 32 / BS + i, last_blk, NB);
        const char* src = (part == 0 ? kpool : vpool) + (size_t)id * bstride + (size_t)g * St::kTile +
                          (size_t)(w % tileU) * 16;
        r[k] = *(const u32x4*)src;
      }
    }
  }

  // Copy into LDS.  nvalid = tokens of the chunk before the sequence's end: on
  // the chunk holding the end (nvalid < 32, uniform) the V elements of later
  // tokens are zeroed, since a P of 0 does not cancel whatever the pool holds
  // there (K needs nothing: masked scores are selected, not multiplied).
  __device__ __forceinline__ void store(char* lds, int tid, int nvalid) const {
    constexpr int tileU = St::kTile / 16;
    constexpr int E = 16 / St::S;  // elements per 16-byte unit
    static_assert(St::S <= 2, "prefill pools hold bf16 or E4M3");
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int u = tid + k * NT;
      if (St::kUnits % NT == 0 || u < St::kUnits) {
        u32x4 v = r[k];
        if (nvalid < 32 && u >= St::NBCH * tileU) {  // a V unit of the chunk holding the end
          const int w = u - St::NBCH * tileU;
          const int tok0 = (w / tileU) * BS, e0 = (w % tileU) * E;  // tile [D][BS]: element e is token e % BS
#pragma unroll
          for (int j = 0; j < E; ++j)
            if (tok0 + (e0 + j) % BS >= nvalid) v[j * St::S / 4] &= ~(((1u << (8 * St::S)) - 1u) << (8 * ((j * St::S) % 4)));
        }
        *(u32x4*)(lds + (size_t)u * 16) = v;
      }
    }
  }
};

// online softmax update of one column tile (S^T already computed): rescales
// acc when the running maximum moves and returns P as bf16 hi + lo operands.
// sl >= 0 (a negative scale is folded into the sign of q).  The causal mask
// is applied only on chunks that reach past some column's position (diag,
// wave-uniform, marked unlikely so that the compiler branches around it
// rather than computing both forms): masked keys are left out of the maximum
// and their P is selected to 0 after the exponential, which also holds for
// sl = 0 and for whatever the pool holds past the sequence's end.
template <int D>
__device__ __forceinline__ void softmax_p(const f32x4 (&s)[2], f32x4 (&acc)[D / 16], float& m, float& l, int cs,
                                          int p_lane, bool diag, float sl, int lane, u32x4& ph, u32x4& pl) {
  const int kg = lane >> 4;
  float cm = -INFINITY;
  if (__builtin_expect(diag, 0)) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) cm = fmaxf(cm, cs + 16 * a + 4 * kg + i <= p_lane ? s[a][i] : -INFINITY);
  } else {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) cm = fmaxf(cm, s[a][i]);
  }
  cm = max_over_groups(cm) * sl;  // the chunk's scaled maximum of the column (log2 units)
  const bool need = cm > m + kRescaleLog2;
  if (__ballot(need)) {
    const float mu = need ? cm : m;
    const float alpha = exp2_fast(m - mu);
    l *= alpha;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float ai = __shfl(alpha, 4 * kg + i, 64);
#pragma unroll
      for (int t = 0; t < D / 16; ++t) acc[t][i] *= ai;
    }
    m = mu;
  }
  float p[8];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int i = 0; i < 4; ++i) p[4 * a + i] = exp2_fast(fmaf(s[a][i], sl, -m));  // key 0 is in every column's range: m is finite
  if (__builtin_expect(diag, 0)) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) p[4 * a + i] = cs + 16 * a + 4 * kg + i <= p_lane ? p[4 * a + i] : 0.f;
  }
  l += ((p[0] + p[1]) + (p[2] + p[3])) + ((p[4] + p[5]) + (p[6] + p[7]));
  uint32_t hb[8];
  float lo[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const uint32_t bits = __builtin_bit_cast(uint32_t, p[j]);
    hb[j] = bits;
    lo[j] = p[j] - __builtin_bit_cast(float, bits & 0xFFFF0000u);
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    ph[w] = __builtin_amdgcn_perm(hb[2 * w + 1], hb[2 * w], 0x07060302u);
    pl[w] = __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, lo[2 * w + 1]),
                                  __builtin_bit_cast(uint32_t, lo[2 * w]), 0x07060302u);
  }
  ph = tokens_by_eight(ph);
  pl = tokens_by_eight(pl);
}

// O += P V over one staged chunk for R tiles: each V operand (8 consecutive
// tokens of one column per lane) is read once from LDS for all tiles.
template <int D, int BS, int KVT, int R>
__device__ __forceinline__ void pv_chunk(const char* vb, const u32x4 (&ph)[R], const u32x4 (&pl)[R],
                                         f32x4 (&acc)[R][D / 16]) {
  using St = Stage<D, BS, KVT>;
  constexpr int S = St::S;
#pragma unroll
  for (int t = 0; t < D / 16; ++t) {
    u32x4 vop;
    if constexpr (KVT == PKV_BF16) {
      vop = *(const u32x4*)(vb + (size_t)t * 16 * BS * S);
    } else {
      const u32x2 w = *(const u32x2*)(vb + (size_t)t * 16 * BS * S);
      vop = e4m3x8_to_bf16x8(w.x, w.y);
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      acc[r][t] = mfma16x16x32(ph[r], vop, acc[r][t]);
      acc[r][t] = mfma16x16x32(pl[r], vop, acc[r][t]);
    }
  }
}

// one wave's R column tiles over one staged chunk: every K and V operand read
// from LDS serves all R tiles
template <int D, int BS, int KVT, int R>
__device__ __forceinline__ void prefill_chunk(const char* lds, const u32x4 (&qop)[R][D / 32],
                                              f32x4 (&acc)[R][D / 16], float (&m)[R], float (&l)[R], int chunk,
                                              const int (&p_lane)[R], int p_min, float sl, int lane) {
  using St = Stage<D, BS, KVT>;
  constexpr int S = St::S;
  const int cs = chunk * 32;
  const int mrow = lane & 15, kg = lane >> 4;
  const char* kl = lds;
  const char* vl = lds + St::NBCH * St::kTile;
  // wave-uniform: some key of the chunk lies past the earliest query position of the wave
  const bool diag = cs + 31 > p_min;
  // ---- S^T = K Q^T for the two 16-token halves, every tile
  f32x4 s[R][2];
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const int tk = 16 * a + mrow;
    const char* kb = kl + (BS >= 32 ? 0 : (tk / BS) * St::kTile) + (size_t)(kg * BS + tk % BS) * 16;
#pragma unroll
    for (int r = 0; r < R; ++r) s[r][a] = f32x4{0.f, 0.f, 0.f, 0.f};
    if constexpr (KVT == PKV_BF16) {
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const u32x4 kop = *(const u32x4*)(kb + (size_t)c * 64 * BS);
#pragma unroll
        for (int r = 0; r < R; ++r) s[r][a] = mfma16x16x32(kop, qop[r][c], s[r][a]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < D / 64; ++u) {
        const u32x4 w = *(const u32x4*)(kb + (size_t)u * 64 * BS);
        const u32x4 k0 = e4m3x8_to_bf16x8(w.x, w.y), k1 = e4m3x8_to_bf16x8(w.z, w.w);
#pragma unroll
        for (int r = 0; r < R; ++r) {
          s[r][a] = mfma16x16x32(k0, qop[r][2 * u], s[r][a]);
          s[r][a] = mfma16x16x32(k1, qop[r][2 * u + 1], s[r][a]);
        }
      }
    }
  }
  // ---- P of every tile, then each V operand (8 consecutive tokens of one column per lane)
  // read once from LDS for all tiles (V rows past n were zeroed when the chunk was staged)
  u32x4 ph[R], pl[R];
#pragma unroll
  for (int r = 0; r < R; ++r) softmax_p<D>(s[r], acc[r], m[r], l[r], cs, p_lane[r], diag, sl, lane, ph[r], pl[r]);
  const int tv = 8 * kg;
  const char* vb = vl + (BS >= 32 ? 0 : (tv / BS) * St::kTile) + ((size_t)mrow * BS + tv % BS) * S;
  pv_chunk<D, BS, KVT, R>(vb, ph, pl, acc);
}

template <int D, int BS, int KVT, int NW, int R>
__global__ __launch_bounds__(64 * NW, 2) void prefill_kernel(PrefillArgs a) {
  using St = Stage<D, BS, KVT>;
  constexpr int NT = 64 * NW;
  __shared__ __align__(16) char sh_stage[kStages][St::kBytes];
  const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
  const int G = a.G;
  const int tok_per_tile = 16 / G;
  const int tok_per_wave = R * tok_per_tile;
  const int tok_per_wg = NW * tok_per_wave;
  // ---- work item: XCD-aware deal of (sequence, KV head, tile group), latest tile group first
  const int items = a.items;
  const int per_xcd = (items + 7) / 8;
  const int item = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (item >= items) return;
  const int groups = a.groups_per_seq;  // tile groups of the longest chunk
  const int seg = item / groups;        // (b, g) in sequence-major order
  const int b = seg / a.H_kv, g = seg % a.H_kv;
  const int q0 = a.query_start[b], C = a.query_start[b + 1] - q0;
  // rows outside the T query rows the host declared are never touched (caller error)
  if (q0 < 0 || C <= 0 || q0 + C > a.T) return;
  const int grp = groups - 1 - item % groups;  // latest first
  const int tok0 = grp * tok_per_wg;
  if (tok0 >= C) return;
  const int n = uniform(min(max(a.context_lens[b], 0), a.len_cap));
  if (n < C) {  // caller error (the chunk is longer than the sequence): zero rows, nothing read
    for (int e = tid; e < min(tok_per_wg, C - tok0) * G * D; e += NT) {
      const int r = e / (G * D);
      a.out[((size_t)(q0 + tok0 + r) * a.H_q + g * G) * D + e % (G * D)] = 0.f;
    }
    return;
  }
  const int last_blk = (n + BS - 1) / BS - 1;
  const int32_t* tab = a.block_tables + (size_t)b * a.max_blocks;
  // this workgroup's queries: positions n - C + tok0 .. ; its last chunk covers the latest one
  const int p_wg_max = n - C + min(C, tok0 + tok_per_wg) - 1;
  const int nch = p_wg_max / 32 + 1;
  // ---- this wave's R column tiles: tile r, column c = (token wtok0 + r * tok_per_tile + c / G, head c % G)
  const int col = lane & 15, kgq = lane >> 4;
  const int wtok0 = tok0 + w * tok_per_wave;
  const int p_min = uniform(n - C + min(wtok0, C - 1));
  // scores in log2 units: (q . k) * sl; a negative sl is taken as |sl| with q negated
  // (a sign flip of each bf16, exact), so that the chunk maximum can be taken before scaling
  float sl = a.scale_log2;
  if constexpr (KVT == PKV_FP8_E4M3) sl *= a.k_scale[g];
  const uint32_t qsign = sl < 0.f ? 0x80008000u : 0u;
  sl = fabsf(sl);
  u32x4 qop[R][D / 32];
  int p_lane[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int qtok = wtok0 + r * tok_per_tile + col / G;  // chunk-relative token of this lane's column
    const bool qvalid = qtok < C;
    p_lane[r] = n - C + (qvalid ? qtok : min(wtok0, C - 1));  // never past the sequence
    const uint16_t* qrow =
        (const uint16_t*)a.q + ((size_t)(q0 + (qvalid ? qtok : 0)) * a.H_q + g * G + col % G) * D;
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (qvalid) v = *(const u32x4*)(qrow + qk_dofs<KVT>(c, kgq));
      qop[r][c] = v ^ qsign;
    }
  }
  f32x4 acc[R][D / 16];
  float m[R], l[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
#pragma unroll
    for (int t = 0; t < D / 16; ++t) acc[r][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[r] = -INFINITY;
    l[r] = 0.f;
  }
  // ---- pipeline: iteration c first writes chunk c+1 (loaded into registers during
  // iteration c-1) into the LDS buffer chunk c-1 used, then reuses those registers for the
  // loads of chunk c+2, then computes chunk c; the barrier closes both buffers' hand-over
  const char* kpool = (const char*)a.k_pool;
  const char* vpool = (const char*)a.v_pool;
  Stager<D, BS, KVT, NT> A;
  A.load(kpool, vpool, tab, 0, last_blk, a.NB, a.H_kv, g, tid);
  A.store(sh_stage[0], tid, n);
  if (nch > 1) A.load(kpool, vpool, tab, 1, last_blk, a.NB, a.H_kv, g, tid);
  __syncthreads();
  for (int c = 0; c < nch; ++c) {
    if (c + 1 < nch) {
      A.store(sh_stage[(c + 1) % kStages], tid, n - 32 * (c + 1));
      if (c + 2 < nch) A.load(kpool, vpool, tab, c + 2, last_blk, a.NB, a.H_kv, g, tid);
    }
    prefill_chunk<D, BS, KVT, R>(sh_stage[c % kStages], qop, acc, m, l, c, p_lane, p_min, sl, lane);
    __syncthreads();
  }
  // ---- normalise and write this wave's rows (row i of tile r = column i of that tile)
  const float vs = KVT == PKV_FP8_E4M3 ? a.v_scale[g] : 1.f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float lt = l[r];
    lt += __shfl_xor(lt, 16, 64);
    lt += __shfl_xor(lt, 32, 64);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * kgq + i;
      const float lr = __shfl(lt, row, 64);
      const int rt = wtok0 + r * tok_per_tile + row / G;
      if (rt < C) {
        float* orow = a.out + ((size_t)(q0 + rt) * a.H_q + g * G + row % G) * D;
#pragma unroll
        for (int t = 0; t < D / 16; ++t) orow[16 * t + col] = acc[r][t][i] * vs / lr;
      }
    }
  }
}

constexpr int kPrefillWaves = 8;
constexpr int kPrefillTiles = 1;  // column tiles per wave (2 measured the same: the loop is VALU-bound)

template <int D, int BS, int KVT>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t s) {
  hipLaunchKernelGGL((prefill_kernel<D, BS, KVT, kPrefillWaves, kPrefillTiles>),
                     dim3((unsigned)((a.items + 7) / 8 * 8)), dim3(64 * kPrefillWaves), 0, s, a);
  return hipGetLastError();
}

template <int D, int KVT>
hipError_t launch_prefill_bs(const PrefillArgs& a, hipStream_t s) {
  switch (a.bs) {
    case 8: return launch_prefill_t<D, 8, KVT>(a, s);
    case 16: return launch_prefill_t<D, 16, KVT>(a, s);
    default: return launch_prefill_t<D, 32, KVT>(a, s);
  }
}

}  // namespace

int prefill_wg_tokens(int G) { return kPrefillWaves * kPrefillTiles * (16 / G); }

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  if (a.kv_dtype == PKV_BF16)
    return a.D == 64 ? launch_prefill_bs<64, PKV_BF16>(a, s) : launch_prefill_bs<128, PKV_BF16>(a, s);
  return a.D == 64 ? launch_prefill_bs<64, PKV_FP8_E4M3>(a, s) : launch_prefill_bs<128, PKV_FP8_E4M3>(a, s);
}

}  // namespace pkv
