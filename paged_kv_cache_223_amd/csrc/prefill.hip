// Paged prefill (chunked multi-query attention) for gfx950 (CDNA4).
//
// Method: "Paged Attention and KV Cache Fragmentation" (inferenceengineering.co),
// section "How PagedAttention maps an OS concept onto GPU memory": a sequence
// takes blocks as it grows; a prompt, or each chunk of it, is appended into
// them and then attends, causally, over everything before it through the
// same block table the decode walks.  Query i of the C_b new tokens of
// sequence b sits at position p = n_b - C_b + i and attends positions 0..p.
//
// Tiles.  A wave owns 32 columns: 32 (query token, head) pairs of one KV head
// g, i.e. 32 / G consecutive query tokens times the G query heads sharing g.
// Per 32-key chunk it runs, on v_mfma_f32_32x32x16_bf16,
//     S^T[32 keys][32 cols] = K[32 keys][D] . Q^T[D][32 cols]        (D/16 MFMAs)
//     O^T[D][32 cols]     += V^T[D][32 keys] . P^T[32 keys][32 cols] (2 D/16 MFMAs)
// With keys as the rows of S^T and columns in lanes, a lane holds 16 scores of
// one column: the chunk maximum is 15 maxima in the lane and one exchange with
// lane l ^ 32, and the accumulator rows a lane holds in O^T belong to the same
// column, so the online-softmax rescale is lane-local.  PV runs in fp16 on
// v_mfma_f32_32x32x16_f16: P rounded to fp16 (a single bf16 P would exceed a
// 2e-3 relative row error on short contexts) and V staged as fp16, exact for
// E4M3 and for bf16 up to 65280 in magnitude; a workgroup whose bf16 V holds a
// larger value runs again with the pool's bf16 V and P as bf16 hi + lo parts
// (two MFMAs each).  P is regrouped with four v_permlane32_swap so that lane
// group h holds keys 8h .. 8h+7 of each 16-key half, which V^T's operand (8
// consecutive keys of one head-dim row) matches.
//
// Workgroups.  NW = 12 waves (three per SIMD at about 165 VGPRs) cover
// NW * 32 / G consecutive query tokens of one (sequence, KV head); measured on
// the 70B layer shape, 12 waves beat 8 and 4, and a software-pipelined loop
// (the next chunk's QK^T under this chunk's softmax) lost for want of
// registers.  Where 12-wave workgroups would leave compute units idle (few
// work items: small batches, small G), the host launches 8-wave ones; each
// wave's columns and chunks are the same either way.  They share every 32-key K/V chunk through LDS.  E4M3 pools: the
// workgroup copies a chunk's pool tiles through registers into one of two LDS
// buffers while the waves compute the previous chunk from the other, with the
// chunk after that already loading into registers.  bf16 pools: K tiles go
// straight from the pool into LDS (global_load_lds_dwordx4) two chunks ahead,
// into the third of three buffers, and only V passes through registers.  The
// LDS copy is laid out for the operand reads, without bank conflicts: K as bf16
// [D/8][32 keys][8 elements] (E4M3 codes decoded once, while staging, rather
// than by each of the 12 waves that read them), V as [D][32 keys] two-byte rows
// padded to 80 bytes.  Work items are dealt to the 8 XCDs so that the workgroups of
// one (sequence, KV head) share one XCD's L2, latest (longest) tiles first.

#include <hip/hip_runtime.h>

#include <math.h>

#include <type_traits>

#include "internal.h"
#include "tile_ops.h"

namespace pkv {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));


__device__ __forceinline__ f32x16 mfma32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ f32x16 mfma32_f16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32); x in the low half
__device__ __forceinline__ uint32_t pack_bf16_rne(float x, float y) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{x, y}), bf16x2));
}


constexpr int kOutStride = 36;  // floats per row of the epilogue tile (16-byte rows, 4-bank shift)

// One 32-key chunk in LDS.  V holds two-byte elements: fp16 on the fast pass, the raw bf16 on the
// rerun of a workgroup whose V does not fit fp16.
template <int D, int BS, int KVT>
struct Stage {
  static constexpr int S = KvTraits<KVT>::kBytes;
  static constexpr int NBCH = BS >= 32 ? 1 : 32 / BS;  // blocks of one chunk
  static constexpr int kTile = D * BS * S;             // one block's tile of one head (K or V) in the pool
  static constexpr int kKBytes = 32 * D * 2;           // K as bf16: [D/8][32][8 elements]
  static constexpr int kVRow = 32 * 2 + 16;            // V row of 32 two-byte elements, padded (bank spread)
  static constexpr int kBytes = kKBytes + D * kVRow;
  static constexpr int kUnits = 2 * NBCH * kTile / 16;  // 16-byte pool units of the chunk (K then V)
};

// Eight bf16 (a 16-byte unit) -> eight fp16, exact for every finite magnitude up to 65280 (the
// largest bf16 value below fp16's maximum; larger ones would become infinities).  Returns the
// largest magnitude in the unit (NaNs ignored: they stay NaNs in fp16) for the range check.
__device__ __forceinline__ float bf16x8_to_f16x8(const u32x4& v, u32x4& h) {
  float lo[4], hi[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = v[i];
    lo[i] = __builtin_bit_cast(float, w << 16);
    hi[i] = __builtin_bit_cast(float, w & 0xFFFF0000u);
    h[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo[i], hi[i]}), f16x2));
  }
  const float m0 = fmaxf(fmaxf(fabsf(lo[0]), fabsf(hi[0])), fabsf(lo[1]));
  const float m1 = fmaxf(fmaxf(m0, fabsf(hi[1])), fabsf(lo[2]));
  const float m2 = fmaxf(fmaxf(m1, fabsf(hi[2])), fabsf(lo[3]));
  return fmaxf(m2, fabsf(hi[3]));
}

// ids[idx] for a lane-dependent idx < N, as selects between scalars (an indexed read of the local
// array would put it in scratch memory).
template <int N>
__device__ __forceinline__ int pick_id(const int (&ids)[N], int idx) {
  int r = ids[0];
#pragma unroll
  for (int i = 1; i < N; ++i) r = idx == i ? ids[i] : r;
  return r;
}

// Copies one chunk's pool tiles (global -> registers -> LDS); the workgroup's threads take
// 16-byte units round-robin.  Blocks past the sequence's last block read the last block again
// (masked later), so every access stays inside the pool.
template <int D, int BS, int KVT, int NT>
struct Stager {
  using St = Stage<D, BS, KVT>;
  static constexpr int kPer = (St::kUnits + NT - 1) / NT;
  static constexpr int tileU = St::kTile / 16;
  u32x4 r[kPer];

  // Table entries of one chunk's blocks (wave-uniform, scalar loads), clamped to the sequence's
  // last block and to the pool.  Taken one iteration ahead of the chunk's loads, so the table's
  // latency is off the loop's critical path.  The table is read through the constant address
  // space (the kernel never writes it), which keeps these loads scalar next to the direct-to-LDS
  // copies (whose memory writes would otherwise make the compiler load them per lane and wait
  // for every copy in flight).
  __device__ __forceinline__ static void chunk_ids(int (&ids)[St::NBCH], const int32_t* __restrict__ tab, int chunk,
                                                   int last_blk, int NB) {
    const __attribute__((address_space(4))) int32_t* ct = (const __attribute__((address_space(4))) int32_t*)tab;
#pragma unroll
    for (int j = 0; j < St::NBCH; ++j) {
      const int jj = min(chunk * 32 / BS + j, last_blk);
      const int id = ct[jj];
      ids[j] = (unsigned)id < (unsigned)NB ? id : 0;
    }
  }

  // Pool address of unit u (K units first, then V) of the chunk whose block ids are ids.
  __device__ __forceinline__ static const char* unit_src(const char* __restrict__ kpool,
                                                         const char* __restrict__ vpool, const int (&ids)[St::NBCH],
                                                         int H_kv, int g, int u) {
    const int part = u / (St::NBCH * tileU);  // 0 = K, 1 = V
    const int w = u % (St::NBCH * tileU);
    const int id = pick_id<St::NBCH>(ids, w / tileU);
    return (part == 0 ? kpool : vpool) + (size_t)id * ((size_t)H_kv * St::kTile) + (size_t)g * St::kTile +
           (size_t)(w % tileU) * 16;
  }

  __device__ __forceinline__ void load(const char* __restrict__ kpool, const char* __restrict__ vpool,
                                       const int (&ids)[St::NBCH], int H_kv, int g, int tid) {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int u = tid + k * NT;
      if (St::kUnits % NT == 0 || u < St::kUnits) r[k] = *(const u32x4*)unit_src(kpool, vpool, ids, H_kv, g, u);
    }
  }

  // Into the LDS layout.  nvalid = keys of the chunk before the sequence's end: on the chunk
  // holding the end (nvalid < 32) V elements of later keys are zeroed, since a P of 0 does not
  // cancel whatever the pool holds there (K needs nothing: masked scores are selected, not
  // multiplied).  V goes in as fp16, or (RAW) as the pool's bf16; a bf16 value that fp16 cannot
  // hold sets *beyond.
  template <bool RAW>
  __device__ __forceinline__ void store(char* lds, int tid, int nvalid, int* beyond) const {
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
      const int u = tid + k * NT;
      if (St::kUnits % NT == 0 || u < St::kUnits) {
        if (nvalid < 32)
          put<RAW, true>(lds, u, r[k], nvalid, beyond);
        else
          put<RAW, false>(lds, u, r[k], nvalid, beyond);
      }
    }
  }

  // MASK: the chunk holds the sequence's end (nvalid < 32), a separate copy of the code so that
  // the other chunks carry none of the masking.
  template <bool RAW, bool MASK>
  __device__ __forceinline__ static void put(char* lds, int u, u32x4 v, int nvalid, int* beyond) {
    constexpr int S = St::S;
    constexpr int E = 16 / S;  // elements per 16-byte unit
    const int part = u / (St::NBCH * tileU);
    const int w = u % (St::NBCH * tileU);
    const int blk = w / tileU, e0 = (w % tileU) * E;  // first element of the unit inside the block's tile
    if (part == 0) {
      // pool K tile [D/E][BS][E]: unit (dg, t) holds E dims of key blk * BS + t
      const int dg = e0 / (BS * E), t = (e0 / E) % BS, key = blk * BS + t;
      if constexpr (S == 2) {
        *(u32x4*)(lds + ((size_t)dg * 32 + key) * 16) = v;
      } else {  // 16 dims, decoded to bf16 (exact) -> planes 2 dg (dims 0-7) and 2 dg + 1 (8-15)
        *(u32x4*)(lds + ((size_t)(2 * dg) * 32 + key) * 16) = e4m3x8_to_bf16x8(v.x, v.y);
        *(u32x4*)(lds + ((size_t)(2 * dg + 1) * 32 + key) * 16) = e4m3x8_to_bf16x8(v.z, v.w);
      }
    } else {
      // pool V tile [D][BS]: unit holds E consecutive elements starting at (d, t0)
      char* vb = lds + St::kKBytes;
      if constexpr (MASK) {
#pragma unroll
        for (int j = 0; j < E; ++j) {
          const int key = blk * BS + (e0 + j) % BS;
          if (key >= nvalid) v[j * S / 4] &= ~(((1u << (8 * S)) - 1u) << (8 * ((j * S) % 4)));
        }
      }
      if constexpr (S == 2) {
        if constexpr (BS >= 8) {  // a unit is 8 keys of one row
          const int d = e0 / BS, t0 = e0 % BS;
          u32x4 h = v;
          if constexpr (!RAW) {
            if (bf16x8_to_f16x8(v, h) > 65280.f) *beyond = 1;
          }
          *(u32x4*)(vb + (size_t)d * St::kVRow + (size_t)(blk * BS + t0) * 2) = h;
        }
      } else {
        const u32x4 h0 = e4m3x8_to_f16x8(v.x, v.y), h1 = e4m3x8_to_f16x8(v.z, v.w);  // codes 0-7, 8-15
        if constexpr (BS == 8) {  // a unit is two rows of 8 keys
          const int d = e0 / 8;
          *(u32x4*)(vb + (size_t)d * St::kVRow + (size_t)blk * 16) = h0;
          *(u32x4*)(vb + (size_t)(d + 1) * St::kVRow + (size_t)blk * 16) = h1;
        } else {  // 16 keys of one row
          const int d = e0 / BS, t0 = e0 % BS;
          char* p = vb + (size_t)d * St::kVRow + (size_t)(blk * BS + t0) * 2;
          *(u32x4*)p = h0;
          *(u32x4*)(p + 16) = h1;
        }
      }
    }
  }
};

typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;

// bf16 pools: a chunk's K tiles go from the pool straight into LDS (global_load_lds_dwordx4: 16
// bytes per lane, 1 KiB of LDS per wave and instruction, neither registers nor LDS stores; the
// bf16 K layout [D/8][32 keys][8 elements] is that instruction's lane order), and its V units,
// which are converted to fp16 on the way, through one register unit in each of the last 4 D
// threads.  The K copy lands asynchronously: a wave waits for its own copies (s_waitcnt vmcnt)
// before the barrier that publishes the chunk.
template <int D, int BS, int NT>
struct SplitStager {
  using Sg = Stager<D, BS, PKV_BF16, NT>;
  using St = Stage<D, BS, PKV_BF16>;
  static constexpr int kKWaves = St::kKBytes / 1024;  // waves that copy K, one instruction each
  static constexpr int kVUnits = St::kUnits / 2;      // 16-byte V units of a chunk (4 D)
  static constexpr int kV0 = NT - kVUnits;            // first thread that carries a V unit
  static_assert(kKWaves * 64 <= NT && kVUnits <= NT && kV0 % 64 == 0, "chunk copy does not fit the workgroup");
  u32x4 r;

  __device__ __forceinline__ static void copy_k(char* lds, const char* __restrict__ kpool, const int (&ids)[St::NBCH],
                                                int H_kv, int g, int w, int lane) {
    if (w < kKWaves) {  // units 64 w + lane: (dg, key) = ((64 w + lane) / 32, lane % 32)
      const char* src = Sg::unit_src(kpool, kpool, ids, H_kv, g, k_unit(64 * w + lane));
      __builtin_amdgcn_global_load_lds((global_void_ptr)src, (lds_void_ptr)(lds + 1024 * w), 16, 0, 0);
    }
  }

  // pool unit of LDS K slot L = dg * 32 + key: unit (blk, dg, t) = blk * tileU + dg * BS + t
  __device__ __forceinline__ static int k_unit(int L) {
    const int dg = L >> 5, key = L & 31;
    return (key / BS) * Sg::tileU + dg * BS + key % BS;
  }

  __device__ __forceinline__ void load_v(const char* __restrict__ kpool, const char* __restrict__ vpool,
                                         const int (&ids)[St::NBCH], int H_kv, int g, int tid) {
    if (tid >= kV0) r = *(const u32x4*)Sg::unit_src(kpool, vpool, ids, H_kv, g, kVUnits + tid - kV0);
  }

  template <bool RAW>
  __device__ __forceinline__ void store_v(char* lds, int tid, int nvalid, int* beyond) const {
    if (tid >= kV0) {
      if (nvalid < 32)
        Sg::template put<RAW, true>(lds, kVUnits + tid - kV0, r, nvalid, beyond);
      else
        Sg::template put<RAW, false>(lds, kVUnits + tid - kV0, r, nvalid, beyond);
    }
  }

  // vector-memory loads this wave issues per chunk (K copy, V unit)
  __device__ __forceinline__ static int loads_per_chunk(int w) { return (w < kKWaves) + (64 * w >= kV0); }
};

// Workgroup barrier after this wave's LDS stores: s_waitcnt lgkmcnt(0), s_barrier, and no
// reordering of memory accesses across it.  __syncthreads() would also wait for every
// direct-to-LDS copy in flight, including those of chunks read two iterations later.
__device__ __forceinline__ void barrier_lds() { __asm__ volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// s_waitcnt vmcnt(n) for a wave-uniform n <= 2 (expcnt and lgkmcnt left alone)
__device__ __forceinline__ void wait_vmcnt(int n) {
  if (n <= 0)
    __builtin_amdgcn_s_waitcnt(0xF70);
  else if (n == 1)
    __builtin_amdgcn_s_waitcnt(0xF71);
  else
    __builtin_amdgcn_s_waitcnt(0xF72);
}

// Regroup one P part for the PV MFMAs.  In: lane (col, h) holds packed bf16 pairs w[k] of keys
// 8 (k / 2) + 4 h + 2 (k % 2) + {0, 1} (the S^T accumulator rows).  Out: op[a] holds keys
// 16 a + 8 h .. 16 a + 8 h + 7 in order, the B operand of the a-th 16-key half.
// permlane32_swap(x, y) leaves lanes 0-31 of x and lanes 32-63 of y in place and exchanges
// x's lanes 32-63 with y's lanes 0-31.
__device__ __forceinline__ void regroup_p(const uint32_t (&w)[8], u32x4 (&op)[2]) {
#pragma unroll
  for (int a = 0; a < 2; ++a) {
    const auto s0 = __builtin_amdgcn_permlane32_swap(w[4 * a], w[4 * a + 2], false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(w[4 * a + 1], w[4 * a + 3], false, false);
    const uint32_t x0 = s0[0], y0 = s0[1], x1 = s1[0], y1 = s1[1];
    op[a] = u32x4{x0, x1, y0, y1};
  }
}

// S^T[32 keys][32 cols] = K Q^T over one staged chunk: MFMA u covers dims 16 u + 8 h + j in lane
// group h; lane (key, h) holds rows 8 (i / 4) + 4 h + i % 4 of its column.
template <int D>
__device__ __forceinline__ f32x16 chunk_scores(const char* lds, const u32x4 (&qop)[D / 16], int lane) {
  const int key = lane & 31, h = lane >> 5;
  f32x16 s = {};
#pragma unroll
  for (int u = 0; u < D / 16; ++u) {
    const u32x4 kop = *(const u32x4*)(lds + ((size_t)(2 * u + h) * 32 + key) * 16);
    s = mfma32(kop, qop[u], s);
  }
  return s;
}

// Online-softmax step of the lane's column over one chunk: the chunk maximum (keys past the
// column's position left out on a diagonal chunk), the running maximum m moved only when the
// chunk exceeds it by more than 8 in log2 units (then alpha = 2^(m_old - m_new) rescales l here,
// and the accumulator at the caller before this chunk's PV), and P = 2^(s sl - m), 0 for masked
// keys.  sl >= 0.  Returns whether any lane moved its maximum.
template <bool DIAG>
__device__ __forceinline__ bool chunk_exp(const f32x16& s, float& m, float& l, float& alpha, float (&p)[16], int cs,
                                          int p_lane, float sl, int lane) {
  const int h = lane >> 5;
  float cm = -INFINITY;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const bool keep = !DIAG || cs + 8 * (i / 4) + 4 * h + (i % 4) <= p_lane;
    cm = fmaxf(cm, keep ? s[i] : -INFINITY);
  }
  // Off the diagonal, when no lane's own maximum passes m + 8 neither does any column's, so m,
  // l and the accumulator stay as they are and the exchange and the rescale factor are skipped.
  bool moved = false;
  if (DIAG || __ballot(cm * sl > m + kRescaleLog2) != 0ull) {
    {  // with lane l ^ 32 (the column's other 16 keys)
      const uint32_t u = __builtin_bit_cast(uint32_t, cm);
      const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      const uint32_t r0 = r[0], r1 = r[1];
      cm = fmaxf(__builtin_bit_cast(float, r0), __builtin_bit_cast(float, r1));
    }
    cm *= sl;
    const bool need = cm > m + kRescaleLog2;
    const float mu = need ? cm : m;
    alpha = exp2_fast(m - mu);  // 1 where the maximum stays (0 on the first chunk: m = -inf)
    l *= alpha;
    m = mu;
    moved = __ballot(need) != 0ull;
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) {  // key 0 is in every column's range: m is finite
    const float e = exp2_fast(fmaf(s[i], sl, -m));
    p[i] = (!DIAG || cs + 8 * (i / 4) + 4 * h + (i % 4) <= p_lane) ? e : 0.f;
  }
  return moved;
}

// P = hi + lo in bf16 (hi truncates p, lo = p - hi rounds to nearest), summed into l, regrouped
// into the PV B operands.
__device__ __forceinline__ void chunk_pack(const float (&p)[16], float& l, u32x4 (&ph)[2], u32x4 (&pl)[2]) {
  float ps[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) ps[j] = (p[4 * j] + p[4 * j + 1]) + (p[4 * j + 2] + p[4 * j + 3]);
  l += (ps[0] + ps[1]) + (ps[2] + ps[3]);
  uint32_t wh[8], wl[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    const uint32_t b0 = __builtin_bit_cast(uint32_t, p[2 * k]), b1 = __builtin_bit_cast(uint32_t, p[2 * k + 1]);
    wh[k] = __builtin_amdgcn_perm(b1, b0, 0x07060302u);
    wl[k] = pack_bf16_rne(p[2 * k] - __builtin_bit_cast(float, b0 & 0xFFFF0000u),
                          p[2 * k + 1] - __builtin_bit_cast(float, b1 & 0xFFFF0000u));
  }
  regroup_p(wh, ph);
  regroup_p(wl, pl);
}

// P as fp16 pairs (round to nearest even: relative error 2^-11, against 2^-8 for one bf16 part),
// regrouped into the PV B operands.  l takes the same fp16 values that PV multiplies, summed in
// fp32 by dot products with (1, 1): eight instructions for the lane's 16 keys instead of 15 adds.
__device__ __forceinline__ void chunk_pack16(const float (&p)[16], float& l, u32x4 (&ph)[2]) {
  uint32_t wh[8];
#pragma unroll
  for (int k = 0; k < 8; ++k)
    wh[k] = pack_f16(p[2 * k], p[2 * k + 1]);
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int k = 0; k < 8; k += 2) {
    s0 = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, wh[k]), one, s0, false);
    s1 = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, wh[k + 1]), one, s1, false);
  }
  l += s0 + s1;
  regroup_p(wh, ph);
}

// O^T += V^T P^T over one staged chunk: A = 8 consecutive keys of one head-dim row (V rows past n
// were zeroed when the chunk was staged).  Fast pass: V and P in fp16, one MFMA per 16-key half.
// RAW (a rerun with the pool's bf16 V): P as bf16 hi + lo, two MFMAs per half.
template <int D, int BS, int KVT, bool RAW>
__device__ __forceinline__ void chunk_pv(const char* lds, const u32x4 (&ph)[2], const u32x4 (&pl)[2],
                                         f32x16 (&acc)[D / 32], int lane) {
  using St = Stage<D, BS, KVT>;
  const int key = lane & 31, h = lane >> 5;
  const char* vb = lds + St::kKBytes;
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
#pragma unroll
    for (int a = 0; a < 2; ++a) {
      const u32x4 vop = *(const u32x4*)(vb + (size_t)(32 * t + key) * St::kVRow + (16 * a + 8 * h) * 2);
      if constexpr (RAW) {
        acc[t] = mfma32(vop, ph[a], acc[t]);
        acc[t] = mfma32(vop, pl[a], acc[t]);
      } else {
        acc[t] = mfma32_f16(vop, ph[a], acc[t]);
      }
    }
  }
}

template <int D, int BS, int KVT, int NW>
__global__ __launch_bounds__(64 * NW, 2) void prefill_kernel(PrefillArgs a) {
  using St = Stage<D, BS, KVT>;
  constexpr int NT = 64 * NW;
  // Chunk buffers: two for E4M3 pools (register copy), three for bf16 pools, whose K copy lands
  // asynchronously two iterations ahead.  Distinct arrays, so that the compiler can tell the
  // buffer being copied into from the one being read and need not wait for the copy before
  // every LDS read.
  __shared__ __align__(16) char sh_b0[St::kBytes];
  __shared__ __align__(16) char sh_b1[St::kBytes];
  __shared__ __align__(16) char sh_b2[KVT == PKV_BF16 ? St::kBytes : 16];
  __shared__ __align__(16) float sh_out[NW * 32 * kOutStride];  // the epilogue's per-wave tiles
  const int tid = threadIdx.x, lane = tid & 63, w = uniform(tid >> 6);
  const int G = a.G;
  const int tok_per_wave = 32 / G;
  const int tok_per_wg = NW * tok_per_wave;
  // ---- work item: XCD-aware deal of (sequence, KV head, token group), latest group first
  const int items = a.items;
  const int per_xcd = (items + 7) / 8;
  const int item = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (item >= items) return;
  const int groups = a.groups_per_seq;  // token groups of the longest chunk
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
  // ---- this wave's 32 columns: column c = (token wtok0 + c / G, head c % G)
  const int col = lane & 31, h = lane >> 5;
  const int wtok0 = tok0 + w * tok_per_wave;
  const int p_min = uniform(n - C + min(wtok0, C - 1));
  const int p_wmax = uniform(n - C + min(wtok0 + tok_per_wave, C) - 1);  // the wave's latest position
  // scores in log2 units: (q . k) * sl; a negative sl is taken as |sl| with q negated
  // (a sign flip of each bf16, exact), so that the chunk maximum can be taken before scaling
  float sl = a.scale_log2;
  if constexpr (KVT == PKV_FP8_E4M3) sl *= a.k_scale[g];
  const uint32_t qsign = sl < 0.f ? 0x80008000u : 0u;
  sl = fabsf(sl);
  const int qtok = wtok0 + col / G;  // chunk-relative token of this lane's column
  const bool qvalid = qtok < C;
  const int p_lane = n - C + (qvalid ? qtok : min(wtok0, C - 1));  // never past the sequence
  u32x4 qop[D / 16];  // B operand of MFMA u: dims 16 u + 8 h .. + 7 of the lane's column
  {
    const uint16_t* qrow = (const uint16_t*)a.q + ((size_t)(q0 + (qvalid ? qtok : 0)) * a.H_q + g * G + col % G) * D;
#pragma unroll
    for (int u = 0; u < D / 16; ++u) {
      u32x4 v = u32x4{0u, 0u, 0u, 0u};
      if (qvalid) v = *(const u32x4*)(qrow + 16 * u + 8 * h);
      qop[u] = v ^ qsign;
    }
  }
  f32x16 acc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};
  float m = -INFINITY, l = 0.f;
  const char* kpool = (const char*)a.k_pool;
  const char* vpool = (const char*)a.v_pool;
  // Fast pass with V and P in fp16.  A bf16 V value that fp16 cannot hold (a magnitude beyond 65280,
  // infinities included; NaNs stay NaNs in fp16) raises sh_beyond while the chunks are staged; the
  // workgroup then runs again with the pool's bf16 V and P as bf16 hi + lo parts, which holds any
  // input (E4M3 values always fit).  The flag is cleared before a barrier that every staging store
  // follows.
  __shared__ int sh_beyond;
  if (tid == 0) sh_beyond = 0;
  __syncthreads();
  using Sg = Stager<D, BS, KVT, NT>;
  // One 32-key chunk of the wave's columns from a staged buffer: S = K Q^T, the online-softmax
  // step, P, O += V^T P^T.
  float p[16], alpha;
  auto compute = [&](auto raw_tag, int c, const char* buf) {
    constexpr bool RAW = decltype(raw_tag)::value;
    if (32 * c > p_wmax) return;
    const f32x16 s = chunk_scores<D>(buf, qop, lane);
    u32x4 ph[2], pl[2];
    const bool moved = 32 * c + 31 > p_min ? chunk_exp<true>(s, m, l, alpha, p, 32 * c, p_lane, sl, lane)
                                           : chunk_exp<false>(s, m, l, alpha, p, 32 * c, p_lane, sl, lane);
    if (moved) {
#pragma unroll
      for (int t = 0; t < D / 32; ++t) acc[t] *= alpha;
    }
    if constexpr (RAW)
      chunk_pack(p, l, ph, pl);
    else
      chunk_pack16(p, l, ph);
    chunk_pv<D, BS, KVT, RAW>(buf, ph, pl, acc, lane);
  };
  auto run = [&](auto raw_tag) {
    constexpr bool RAW = decltype(raw_tag)::value;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};
    m = -INFINITY;
    l = 0.f;
    int ids[St::NBCH];
    if constexpr (KVT == PKV_BF16) {
      // Iteration c: V of chunk c + 1 into its buffer; K of chunk c + 2 copied into the buffer of
      // chunk c - 1 (read up to the previous barrier) and its V loaded; chunk c computed; then
      // this wave's copies older than those of this iteration waited for, and the barrier.
      using Sp = SplitStager<D, BS, NT>;
      Sp A;
      const int per_chunk = Sp::loads_per_chunk(w);
      Sg::chunk_ids(ids, tab, 0, last_blk, a.NB);
      Sp::copy_k(sh_b0, kpool, ids, a.H_kv, g, w, lane);
      A.load_v(kpool, vpool, ids, a.H_kv, g, tid);
      A.template store_v<RAW>(sh_b0, tid, n, &sh_beyond);
      Sg::chunk_ids(ids, tab, 1, last_blk, a.NB);
      if (nch > 1) {
        Sp::copy_k(sh_b1, kpool, ids, a.H_kv, g, w, lane);
        A.load_v(kpool, vpool, ids, a.H_kv, g, tid);
      }
      Sg::chunk_ids(ids, tab, 2, last_blk, a.NB);  // clamped: always inside the table row
      wait_vmcnt(nch > 1 ? per_chunk : 0);
      __syncthreads();
      auto step = [&](int c, const char* cur, char* nx1, char* nx2) {
        if (c + 1 < nch) A.template store_v<RAW>(nx1, tid, n - 32 * (c + 1), &sh_beyond);
        const bool more = c + 2 < nch;
        if (more) {
          Sp::copy_k(nx2, kpool, ids, a.H_kv, g, w, lane);
          A.load_v(kpool, vpool, ids, a.H_kv, g, tid);
          Sg::chunk_ids(ids, tab, c + 3, last_blk, a.NB);
        }
        compute(raw_tag, c, cur);
        wait_vmcnt(more ? per_chunk : 0);
        barrier_lds();
      };
      for (int c = 0; c < nch; c += 3) {
        step(c, sh_b0, sh_b1, sh_b2);
        if (c + 1 < nch) step(c + 1, sh_b1, sh_b2, sh_b0);
        if (c + 2 < nch) step(c + 2, sh_b2, sh_b0, sh_b1);
      }
    } else {
      Sg A;
      Sg::chunk_ids(ids, tab, 0, last_blk, a.NB);
      A.load(kpool, vpool, ids, a.H_kv, g, tid);
      A.template store<RAW>(sh_b0, tid, n, &sh_beyond);
      Sg::chunk_ids(ids, tab, 1, last_blk, a.NB);
      if (nch > 1) A.load(kpool, vpool, ids, a.H_kv, g, tid);
      Sg::chunk_ids(ids, tab, 2, last_blk, a.NB);  // clamped: always inside the table row
      __syncthreads();
      for (int c = 0; c < nch; ++c) {
        if (c + 1 < nch) {
          A.template store<RAW>((c & 1) ? sh_b0 : sh_b1, tid, n - 32 * (c + 1), &sh_beyond);
          if (c + 2 < nch) {
            A.load(kpool, vpool, ids, a.H_kv, g, tid);
            Sg::chunk_ids(ids, tab, c + 3, last_blk, a.NB);
          }
        }
        compute(raw_tag, c, (c & 1) ? sh_b1 : sh_b0);
        __syncthreads();
      }
    }
  };
  // E4M3 pools: fixed wave priorities (waves 8-11 highest, then 4-7; the first 512 threads stage a
  // chunk at D = 128), so that after each barrier the waves of a SIMD do not all issue their
  // QK^T, softmax and PV in step: the first reaches its softmax while the others still use the
  // matrix core (+1.3 % on the 70B shape; with bf16 pools every order measured was slower).
  if constexpr (KVT == PKV_FP8_E4M3) {
    if (w >= 8)
      __builtin_amdgcn_s_setprio(2);
    else if (w >= 4)
      __builtin_amdgcn_s_setprio(1);
  }
  run(std::false_type{});
  if constexpr (KVT == PKV_BF16)
    if (uniform(sh_beyond)) run(std::true_type{});  // every store to sh_beyond was before the last barrier
  // ---- normalise and write the wave's 32 output rows (row c = column c: token wtok0 + c / G,
  // head g G + c % G), through a per-wave LDS tile one 32-dim segment at a time: acc[t] register i
  // of lane (c, h) is dim 32 t + 8 (i / 4) + 4 h + i % 4 of row c; read back, eight lanes cover a
  // row's 128-byte segment, so each store instruction writes 8 whole cache lines instead of 32-byte
  // pieces of 32 rows.  The stores are non-temporal: the output streams past the L2, which then
  // keeps more of the segment's K/V for the other workgroups reading it.
  {
    const uint32_t u = __builtin_bit_cast(uint32_t, l);
    const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const uint32_t r0 = r[0], r1 = r[1];
    l = __builtin_bit_cast(float, r0) + __builtin_bit_cast(float, r1);
  }
  const float f = (KVT == PKV_FP8_E4M3 ? a.v_scale[g] : 1.f) / l;  // lanes of invalid columns: never stored
  const int rows = uniform(min(32, max(0, (C - wtok0) * G)));
  float* tw = sh_out + w * (32 * kOutStride);
  const size_t row0 = (size_t)(q0 + wtok0) * a.H_q + (size_t)g * G;
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
#pragma unroll
    for (int k = 0; k < 4; ++k)
      *(f32x4*)(tw + col * kOutStride + 8 * k + 4 * h) =
          f32x4{acc[t][4 * k] * f, acc[t][4 * k + 1] * f, acc[t][4 * k + 2] * f, acc[t][4 * k + 3] * f};
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int row = 8 * qq + (lane >> 3), ch = lane & 7;
      const f32x4 v = *(const f32x4*)(tw + row * kOutStride + 4 * ch);
      if (row < rows)
        __builtin_nontemporal_store(v, (f32x4*)(a.out + (row0 + (size_t)(row / G) * a.H_q + row % G) * D + 32 * t + 4 * ch));
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }
}

template <int D, int BS, int KVT>
hipError_t launch_prefill_t(const PrefillArgs& a, hipStream_t s) {
  const dim3 grid((unsigned)((a.items + 7) / 8 * 8));
  if (a.nw == 8)
    hipLaunchKernelGGL((prefill_kernel<D, BS, KVT, 8>), grid, dim3(64 * 8), 0, s, a);
  else
    hipLaunchKernelGGL((prefill_kernel<D, BS, KVT, 12>), grid, dim3(64 * 12), 0, s, a);
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

int prefill_wg_tokens(int G, int nw) { return nw * (32 / G); }

hipError_t launch_prefill(const PrefillArgs& a, hipStream_t s) {
  if (a.kv_dtype == PKV_BF16)
    return a.D == 64 ? launch_prefill_bs<64, PKV_BF16>(a, s) : launch_prefill_bs<128, PKV_BF16>(a, s);
  return a.D == 64 ? launch_prefill_bs<64, PKV_FP8_E4M3>(a, s) : launch_prefill_bs<128, PKV_FP8_E4M3>(a, s);
}

}  // namespace pkv
