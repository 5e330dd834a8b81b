// Paged-KV decode attention, vector path (VALU) for gfx950.
//
// Same operation as the matrix-core path ("KV Cache Fragmentation" field guide, section
// "Definition"; "Paged Attention and KV Cache Fragmentation", sections "How PagedAttention maps
// an OS concept onto GPU memory" and "The non-contiguous memory layout PagedAttention introduces
// and its overhead"): every step goes through the block table and the scores stay on chip.  It
// serves the combinations the matrix-core path does not take: fp32 q or KV, G = H_q / H_kv > 16
// and D = 256.  Work is cut into fixed context splits of split_tokens tokens (a multiple of 256);
// a sequence with more than one split leaves partials that split_merge combines.

#include <hip/hip_runtime.h>

#include <math.h>

#include <type_traits>

#include "decode_common.h"
#include "internal.h"
#include "tile_ops.h"

namespace pkv {
namespace {

// ---------------------------------------------------------------------------
// vector path
// ---------------------------------------------------------------------------
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  float mag = e ? ldexpf((float)(8u + m), (int)e - 10) : ldexpf((float)m, -9);
  if (e == 15u && m == 7u) mag = NAN;
  return (c & 0x80u) ? -mag : mag;
}

template <int KVT>
struct KvBytes {
  static constexpr int v = KVT == PKV_F32 ? 4 : KVT == PKV_BF16 ? 2 : 1;
};

__device__ __forceinline__ float load_elem(const void* p, size_t idx, int dt) {
  if (dt == PKV_F32) return ((const float*)p)[idx];
  if (dt == PKV_BF16) return __builtin_bit_cast(float, (uint32_t)((const uint16_t*)p)[idx] << 16);
  return e4m3_value(((const uint8_t*)p)[idx]);
}

// 16 bytes of KV elements -> fp32 (exact): 4 fp32, 8 bf16 or 16 E4M3 codes (through the exact
// E4M3 -> bf16 conversion the matrix-core path uses)
template <int KVT>
__device__ __forceinline__ void unit_to_f32(const u32x4 w, float (&out)[16 / KvBytes<KVT>::v]) {
  if constexpr (KVT == PKV_F32) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      // through a scalar: a bit cast of a vector element read in place has yielded element 0
      const uint32_t e = w[i];
      out[i] = __builtin_bit_cast(float, e);
    }
  } else if constexpr (KVT == PKV_BF16) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __builtin_bit_cast(float, w[i] << 16);
      out[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const u32x4 bf = e4m3x8_to_bf16x8(w[2 * half], w[2 * half + 1]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        out[8 * half + 2 * i] = __builtin_bit_cast(float, bf[i] << 16);
        out[8 * half + 2 * i + 1] = __builtin_bit_cast(float, bf[i] & 0xFFFF0000u);
      }
    }
  }
}

// 8 consecutive tokens of one V row (a [D][bs] tile row, bs >= 8): 32, 16 or 8 bytes
template <int KVT>
struct VGroup {
  static constexpr int W = 2 * KvBytes<KVT>::v;  // 32-bit words
  uint32_t w[W];
  __device__ __forceinline__ void load(const char* p) {
    if constexpr (W == 8) {
      const u32x4 x = __builtin_nontemporal_load((const u32x4*)p), y = __builtin_nontemporal_load((const u32x4*)p + 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = x[i], w[4 + i] = y[i];
    } else if constexpr (W == 4) {
      const u32x4 x = __builtin_nontemporal_load((const u32x4*)p);
#pragma unroll
      for (int i = 0; i < 4; ++i) w[i] = x[i];
    } else {
      const u32x2 x = __builtin_nontemporal_load((const u32x2*)p);
      w[0] = x[0];
      w[1] = x[1];
    }
  }
  __device__ __forceinline__ void to_f32(float (&v)[8]) const {
    if constexpr (KVT == PKV_F32) {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = __builtin_bit_cast(float, w[i]);
    } else if constexpr (KVT == PKV_BF16) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __builtin_bit_cast(float, w[i] << 16);
        v[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xFFFF0000u);
      }
    } else {
      const u32x4 bf = e4m3x8_to_bf16x8(w[0], w[1]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = __builtin_bit_cast(float, bf[i] << 16);
        v[2 * i + 1] = __builtin_bit_cast(float, bf[i] & 0xFFFF0000u);
      }
    }
  }
};

// Wave-wide float maximum and sum (every lane gets the result).
__device__ __forceinline__ float wave_fmax(float x) {
#pragma unroll
  for (int o = 32; o; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ float wave_fsum(float x) {
#pragma unroll
  for (int o = 32; o; o >>= 1) x += __shfl_xor(x, o, 64);
  return x;
}

__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// Vector path (VALU), one wave per (context split, sequence, KV head, group of HG query heads), so
// that K and V are read once for up to HG heads.  Per step of 64 tokens:
//   - scores: lane t scores token t for the group's heads.  Its K row comes in as 16-byte loads,
//     a 64-dim slice at a time; with bf16 q and bf16 or E4M3 KV the products are bf16 pair dot
//     products accumulated in fp32 (v_dot2_f32_bf16; E4M3 codes convert to bf16 exactly), else
//     fp32 FMAs.  q sits in LDS.
//   - online softmax per head with wave reductions; P goes to LDS as bf16 hi + lo parts (about 16
//     bits), or as fp32 for fp32 KV.
//   - PV: lane owns head dims lane + 64 j and reads 8 consecutive tokens of a V row per load; the
//     step's V loads are issued before its scores when they fit in 64 VGPRs.
// Tokens outside the split or in the masked hole weigh 0, and their V elements are zeroed (0 x NaN
// poison would be NaN).
template <int D, int BS, int KVT, int HG, bool QF32>
__global__ __launch_bounds__(64, 2) void decode_vector_kernel(DecodeArgs a) {
  constexpr int S = KvBytes<KVT>::v;
  constexpr int X = 16 / S;   // elements per 16-byte K unit
  constexpr int KU = 64 / X;  // K units per 64-dim slice
  constexpr int DJ = D / 64;  // V rows (head dims) per lane
  constexpr bool kDotQK = KVT != PKV_F32 && !QF32;
  constexpr bool kDotPV = KVT != PKV_F32;
  __shared__ __align__(16) float sh_q[HG][kDotQK ? D / 2 : D];  // bf16 pairs (bits) or fp32
  __shared__ __align__(16) float sh_p[kDotPV ? 2 : 1][HG][64];   // hi, lo bf16 (as halves) or fp32
  const int lane = threadIdx.x;
  const int NG = (a.G + HG - 1) / HG;
  int idx = blockIdx.x;
  const int gi = idx % NG;
  idx /= NG;
  const int g = idx % a.H_kv;
  idx /= a.H_kv;
  const int b = idx % a.B, split = idx / a.B;
  const int n = uniform(seq_len(a.context_lens, b, a.len_cap));
  const int nsplit = n == 0 ? 1 : (n + a.split_tokens - 1) / a.split_tokens;
  if (split >= nsplit) return;
  const int h0 = g * a.G + gi * HG;       // the group's first query head
  const int nh = min(HG, a.G - gi * HG);  // its heads
  if (n == 0) {
    for (int e = lane; e < nh * D; e += 64) a.out[((size_t)b * a.H_q + h0) * D + e] = 0.f;
    return;
  }
  constexpr int bs = BS;
  const int t_begin = split * a.split_tokens;
  const int t_end = min(n, t_begin + a.split_tokens);
  int hlo, hhi;
  seq_hole(a, b, hlo, hhi);
  const int last_blk = (n + bs - 1) / bs - 1;
  const int32_t* tab = a.block_tables + (size_t)b * a.max_blocks;
  if constexpr (kDotQK) {  // bf16 q as it is, in pairs
    const uint32_t* q2 = (const uint32_t*)a.q;
    for (int e = lane; e < HG * D / 2; e += 64) {
      const int hh = e / (D / 2);
      sh_q[hh][e % (D / 2)] =
          __builtin_bit_cast(float, hh < nh ? q2[(((size_t)b * a.H_q + h0 + hh) * D) / 2 + e % (D / 2)] : 0u);
    }
  } else {
    for (int e = lane; e < HG * D; e += 64) {
      const int hh = e / D;
      sh_q[hh][e % D] = hh < nh ? load_elem(a.q, ((size_t)b * a.H_q + h0 + hh) * D + e % D, a.q_dtype) : 0.f;
    }
  }
  __syncthreads();
  float sl = a.scale_log2, vs = 1.f;
  if constexpr (KVT == PKV_FP8_E4M3) {
    sl *= a.k_scale[g];
    vs = a.v_scale[g];
  }
  const size_t tile = (size_t)D * bs * S;  // one head's tile of one block (K or V)
  const size_t bstride = (size_t)a.H_kv * tile;
  const char* kbase = (const char*)a.k_pool + (size_t)g * tile;
  const char* vbase = (const char*)a.v_pool + (size_t)g * tile;
  float m[HG], l[HG], acc[HG][DJ];
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int j = 0; j < DJ; ++j) acc[hh][j] = 0.f;
  }
  // V loads of a step are issued before its scores when they fit in 64 VGPRs at D <= 128 and the
  // scores leave room (bf16 pair dot products, or one head per wave), else group by group in the
  // PV loop
  constexpr bool kPrefetchV = 8 * DJ * VGroup<KVT>::W <= 64 && DJ <= 2 && (kDotQK || HG == 1);
  auto load_v = [&](VGroup<KVT>(&vg)[DJ], int t0, int k) {
    const int tg = min(t0 + 8 * k, t_end - 1);
    const int blk = block_id(tab, tg / bs, last_blk, a.NB);
    const char* vrow = vbase + (size_t)blk * bstride + (tg / 8 * 8 % bs) * S;  // wave-uniform
#pragma unroll
    for (int j = 0; j < DJ; ++j) vg[j].load(vrow + (uint32_t)((lane + 64 * j) * bs * S));
  };
  for (int t0 = t_begin; t0 < t_end; t0 += 64) {
    // q is read from LDS afresh every step: hoisted out of the loop it would take HG x D / 2 VGPRs
    asm volatile("" ::: "memory");
    // wave-uniform: every token of the step is attended
    const bool full = t0 + 64 <= t_end && (t0 + 64 <= hlo || t0 >= hhi);
    VGroup<KVT> vg[kPrefetchV ? 8 : 1][DJ];
    if constexpr (kPrefetchV) {
#pragma unroll
      for (int k = 0; k < 8; ++k) load_v(vg[k], t0, k);
    }
    // ---- scores of the lane's token for the group's heads
    const int tok = t0 + lane;
    const bool valid = tok < t_end && (tok < hlo || tok >= hhi);
    const int tc = min(tok, t_end - 1);
    const char* krow = kbase + (size_t)block_id(tab, tc / bs, last_blk, a.NB) * bstride + (uint32_t)(tc % bs) * 16;
    float sc[HG];
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) sc[hh] = 0.f;
#pragma unroll
    for (int sl64 = 0; sl64 < D / 64; ++sl64) {
      u32x4 ku[KU];
#pragma unroll
      for (int u = 0; u < KU; ++u) ku[u] = __builtin_nontemporal_load((const u32x4*)(krow + (sl64 * KU + u) * bs * 16));
#pragma unroll
      for (int u = 0; u < KU; ++u) {
        const int d0 = (sl64 * KU + u) * X;  // first head dim of the unit
        if constexpr (kDotQK) {
          // bf16 pairs of the unit: 4 (bf16) or 8 (E4M3, through the exact conversion)
          uint32_t kw[X / 2];
          if constexpr (KVT == PKV_BF16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) kw[i] = ku[u][i];
          } else {
            const u32x4 lo = e4m3x8_to_bf16x8(ku[u][0], ku[u][1]), hi = e4m3x8_to_bf16x8(ku[u][2], ku[u][3]);
#pragma unroll
            for (int i = 0; i < 4; ++i) kw[i] = lo[i], kw[4 + i] = hi[i];
          }
#pragma unroll
          for (int hh = 0; hh < HG; ++hh) {
            const u32x4* qv = (const u32x4*)&sh_q[hh][d0 / 2];  // broadcast reads
#pragma unroll
            for (int i4 = 0; i4 < X / 8; ++i4) {
              const u32x4 qq = qv[i4];
#pragma unroll
              for (int i = 0; i < 4; ++i) sc[hh] = dot2_bf16(kw[4 * i4 + i], qq[i], sc[hh]);
            }
          }
        } else {
          float kf[X];
          unit_to_f32<KVT>(ku[u], kf);
#pragma unroll
          for (int hh = 0; hh < HG; ++hh) {
            const f32x4* qv = (const f32x4*)&sh_q[hh][d0];
#pragma unroll
            for (int x4 = 0; x4 < X / 4; ++x4) {
              const f32x4 qq = qv[x4];
#pragma unroll
              for (int x = 0; x < 4; ++x) sc[hh] = fmaf(qq[x], kf[4 * x4 + x], sc[hh]);
            }
          }
        }
      }
    }
    // ---- online softmax per head over the step (wave reductions); probabilities to LDS
    float alpha[HG];
#pragma unroll
    for (int hh = 0; hh < HG; ++hh) {
      const float s = valid ? sc[hh] * sl : -INFINITY;
      const float mn = fmaxf(m[hh], wave_fmax(s));
      alpha[hh] = mn == -INFINITY ? 1.f : exp2_fast(m[hh] - mn);  // nothing attended yet: no rescale
      const float p = valid ? exp2_fast(s - mn) : 0.f;
      l[hh] = l[hh] * alpha[hh] + wave_fsum(p);
      m[hh] = mn;
      if constexpr (kDotPV) {  // hi truncates p, lo = p - hi (both bf16, as fp32 bit patterns' halves)
        const uint32_t bits = __builtin_bit_cast(uint32_t, p);
        const float lo = p - __builtin_bit_cast(float, bits & 0xFFFF0000u);
        ((uint16_t*)sh_p[0][hh])[lane] = (uint16_t)(bits >> 16);
        ((uint16_t*)sh_p[1][hh])[lane] = (uint16_t)(__builtin_bit_cast(uint32_t, lo) >> 16);
      } else {
        sh_p[0][hh][lane] = p;
      }
    }
    __syncthreads();
    // ---- O += P V over the step's 8 groups of 8 tokens
#pragma unroll
    for (int hh = 0; hh < HG; ++hh)
#pragma unroll
      for (int j = 0; j < DJ; ++j) acc[hh][j] *= alpha[hh];
    // one copy of the loop for a fully attended step and one with the token masks (branch-free
    // inside each: per-group branches would split the loop and keep every group's operands live)
    auto pv_step = [&](auto masked) {
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const int tg = t0 + 8 * k;
        if constexpr (!kPrefetchV) load_v(vg[0], t0, k);
#pragma unroll
        for (int j = 0; j < DJ; ++j) {
          const VGroup<KVT>& g8 = vg[kPrefetchV ? k : 0][j];
          if constexpr (kDotPV) {
            // V as bf16 pairs (tokens 2i, 2i + 1 in word i), masked tokens zeroed
            uint32_t vw[4];
            if constexpr (KVT == PKV_BF16) {
#pragma unroll
              for (int i = 0; i < 4; ++i) vw[i] = g8.w[i];
            } else {
              const u32x4 c = e4m3x8_to_bf16x8(g8.w[0], g8.w[1]);
#pragma unroll
              for (int i = 0; i < 4; ++i) vw[i] = c[i];
            }
            if constexpr (decltype(masked)::value) {
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int t = tg + 2 * i;
                const bool ok0 = t < t_end && (t < hlo || t >= hhi);
                const bool ok1 = t + 1 < t_end && (t + 1 < hlo || t + 1 >= hhi);
                vw[i] &= (ok0 ? 0x0000FFFFu : 0u) | (ok1 ? 0xFFFF0000u : 0u);
              }
            }
#pragma unroll
            for (int hh = 0; hh < HG; ++hh) {
              const u32x4 ph = *(const u32x4*)&((const uint16_t*)sh_p[0][hh])[8 * k];
              const u32x4 pl = *(const u32x4*)&((const uint16_t*)sh_p[1][hh])[8 * k];
              float o = acc[hh][j];
#pragma unroll
              for (int i = 0; i < 4; ++i) o = dot2_bf16(ph[i], vw[i], o);
#pragma unroll
              for (int i = 0; i < 4; ++i) o = dot2_bf16(pl[i], vw[i], o);
              acc[hh][j] = o;
            }
          } else {
            float v[8];
            g8.to_f32(v);
            if constexpr (decltype(masked)::value) {
#pragma unroll
              for (int x = 0; x < 8; ++x) {
                const int t = tg + x;
                v[x] = (t < t_end && (t < hlo || t >= hhi)) ? v[x] : 0.f;
              }
            }
#pragma unroll
            for (int hh = 0; hh < HG; ++hh) {
              const f32x4 p0 = *(const f32x4*)&sh_p[0][hh][8 * k], p1 = *(const f32x4*)&sh_p[0][hh][8 * k + 4];
              float o = acc[hh][j];
#pragma unroll
              for (int x = 0; x < 4; ++x) o = fmaf(p0[x], v[x], o);
#pragma unroll
              for (int x = 0; x < 4; ++x) o = fmaf(p1[x], v[4 + x], o);
              acc[hh][j] = o;
            }
          }
        }
      }
    };
    if (full)
      pv_step(std::false_type{});
    else
      pv_step(std::true_type{});
    __syncthreads();
  }
#pragma unroll
  for (int hh = 0; hh < HG; ++hh) {
    if (hh >= nh) break;
    const size_t row = (size_t)b * a.H_q + h0 + hh;
#pragma unroll
    for (int j = 0; j < DJ; ++j) {
      const int d = lane + 64 * j;
      if (nsplit == 1) {
        a.out[row * D + d] = l[hh] > 0.f ? acc[hh][j] * vs / l[hh] : 0.f;  // nothing attended: zero row
      } else {
        const size_t pr = row * a.max_splits + split;
        a.ws_o[pr * D + d] = acc[hh][j] * vs;
        if (d == 0) {
          a.ws_ml[2 * pr] = m[hh];
          a.ws_ml[2 * pr + 1] = l[hh];
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// split merge: one workgroup per (sequence, KV head) with more than one split
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void split_merge_kernel(DecodeArgs a) {
  constexpr int kHeads = 64;  // heads merged per pass
  __shared__ float sh_M[kHeads], sh_iL[kHeads];
  const int b = blockIdx.x / a.H_kv, g = blockIdx.x % a.H_kv;
  const int n = seq_len(a.context_lens, b, a.len_cap);
  const int nsplit = n == 0 ? 1 : (n + a.split_tokens - 1) / a.split_tokens;
  if (nsplit <= 1) return;
  const int D = a.D, tid = threadIdx.x;
  for (int h0 = 0; h0 < a.G; h0 += kHeads) {
    const int nh = min(kHeads, a.G - h0);
    const size_t row0 = (size_t)b * a.H_q + g * a.G + h0;
    if (tid < nh) {
      const float* ml = a.ws_ml + 2 * (row0 + tid) * a.max_splits;
      float M = -INFINITY;
      for (int i = 0; i < nsplit; ++i) M = fmaxf(M, ml[2 * i]);
      float L = 0.f;
      for (int i = 0; i < nsplit; ++i)
        if (ml[2 * i] != -INFINITY) L += exp2_fast(ml[2 * i] - M) * ml[2 * i + 1];
      sh_M[tid] = M == -INFINITY ? 0.f : M;  // nothing attended: zero row
      sh_iL[tid] = L > 0.f ? 1.f / L : 0.f;
    }
    __syncthreads();
    for (int e = tid; e < nh * D; e += 256) {
      const int h = e / D, col = e % D;
      const size_t pr0 = (row0 + h) * a.max_splits;
      const float* ml = a.ws_ml + 2 * pr0;
      const float* o = a.ws_o + pr0 * D + col;
      const float M = sh_M[h];
      float acc = 0.f;
      int i = 0;
      for (; i + 4 <= nsplit; i += 4) {  // four independent loads in flight
        const float o0 = o[(size_t)i * D], o1 = o[(size_t)(i + 1) * D];
        const float o2 = o[(size_t)(i + 2) * D], o3 = o[(size_t)(i + 3) * D];
        acc += exp2_fast(ml[2 * i] - M) * o0 + exp2_fast(ml[2 * i + 2] - M) * o1 +
               exp2_fast(ml[2 * i + 4] - M) * o2 + exp2_fast(ml[2 * i + 6] - M) * o3;
      }
      for (; i < nsplit; ++i) acc += exp2_fast(ml[2 * i] - M) * o[(size_t)i * D];
      a.out[(row0 + h) * D + col] = acc * sh_iL[h];
    }
    __syncthreads();
  }
}

template <int D, int BS, int KVT, int HG, bool QF32>
hipError_t launch_vector_t(const DecodeArgs& a, hipStream_t s) {
  const long long grid = (long long)a.max_splits * a.B * a.H_kv * ((a.G + HG - 1) / HG);
  hipLaunchKernelGGL((decode_vector_kernel<D, BS, KVT, HG, QF32>), dim3((unsigned)grid), dim3(64), 0, s, a);
  return hipGetLastError();
}

template <int D, int BS, int KVT, bool QF32>
hipError_t launch_vector_g(const DecodeArgs& a, hipStream_t s) {
  // fp32 q against E4M3 codes scores in fp32 from 16 converted elements per unit: one head per
  // wave keeps that within the register file (more heads spill)
  if constexpr (KVT == PKV_FP8_E4M3 && QF32) {
    return launch_vector_t<D, BS, KVT, 1, QF32>(a, s);
  } else {
    if (a.G == 1) return launch_vector_t<D, BS, KVT, 1, QF32>(a, s);
    if (a.G == 2) return launch_vector_t<D, BS, KVT, 2, QF32>(a, s);
    return launch_vector_t<D, BS, KVT, 4, QF32>(a, s);  // groups of 4 heads (the last one may be partial)
  }
}

template <int D, int BS, int KVT>
hipError_t launch_vector_q(const DecodeArgs& a, hipStream_t s) {
  if constexpr (KVT == PKV_F32) {
    return launch_vector_g<D, BS, KVT, true>(a, s);
  } else {
    if (a.q_dtype == PKV_BF16) return launch_vector_g<D, BS, KVT, false>(a, s);
    return launch_vector_g<D, BS, KVT, true>(a, s);
  }
}

template <int D, int BS>
hipError_t launch_vector_kv(const DecodeArgs& a, hipStream_t s) {
  switch (a.kv_dtype) {
    case PKV_F32: return launch_vector_q<D, BS, PKV_F32>(a, s);
    case PKV_BF16: return launch_vector_q<D, BS, PKV_BF16>(a, s);
    case PKV_FP8_E4M3: return launch_vector_q<D, BS, PKV_FP8_E4M3>(a, s);
  }
  return hipErrorInvalidValue;
}

template <int D>
hipError_t launch_vector_d(const DecodeArgs& a, hipStream_t s) {
  switch (a.bs) {
    case 8: return launch_vector_kv<D, 8>(a, s);
    case 16: return launch_vector_kv<D, 16>(a, s);
    case 32: return launch_vector_kv<D, 32>(a, s);
  }
  return hipErrorInvalidValue;
}
}  // namespace

hipError_t launch_decode_vector(const DecodeArgs& a, hipStream_t s) {
  switch (a.D) {
    case 64: return launch_vector_d<64>(a, s);
    case 128: return launch_vector_d<128>(a, s);
    case 256: return launch_vector_d<256>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_split_merge(const DecodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(split_merge_kernel, dim3((unsigned)(a.B * a.H_kv)), dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace pkv
