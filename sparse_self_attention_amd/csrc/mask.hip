// Mean-query (pooling) mask for gfx950: group mean -> scores -> per-group cut -> ascending key lists.
//
// FG-Attn review, "The pith" and Referee major comment 2: the queries of a group are averaged,
// every key is scored against the average, and keys with a small pooled score are skipped.
// Chipmunk review, "What carries the argument": alternatively a top-k index mask per chunk.
//
//  k_group_mean   one workgroup per (batch, head, group): fp32 mean of the group's bf16 query rows,
//                 stored as an unevaluated bf16 pair hi + lo (hi = bf16(mean), lo = bf16(mean - hi)),
//                 so the matrix cores score with about 16 mantissa bits of the mean.
//  k_scores       s[g, j] = scale * (hi_g . k_j + lo_g . k_j) with v_mfma_f32_32x32x16_bf16, in tiles
//                 of 32 groups x 32 keys so every K row read feeds 32 groups; fp32 scores of a bounded
//                 number of heads are staged in the workspace (sized to stay in the 256 MB MALL).
//  k_select       one 1024-thread workgroup per group; the group's scores stay in VGPRs when there are
//                 at most 16 per thread, else every pass re-reads them from the L2/MALL-resident stage;
//                 - top-k: finds the k-th largest score by a 3-pass MSB-first radix select
//                   (12 + 12 + 8 bits of an order-preserving integer key) with LDS histograms;
//                   ties at the cut go to the lowest key index;
//                 - threshold: lse by block max + block sum of exp, cut = lse + ln(tau); if nothing
//                   passes, the arg-max key (lowest index on ties) is kept;
//                 then compacts the kept keys into an ascending list: wave ballots + mbcnt give
//                 the in-wave prefix, one block scan over the per-wave counts gives the offsets.
#include <math.h>

#include "../../include/sattn.h"
#include "device_common.hpp"
#include "launch.hpp"

namespace sattn {

constexpr size_t SCORE_STAGE_BUDGET = 320ull << 20;   // bytes of fp32 scores staged per pass
constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;

static inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
// fp32 score rows are padded to a multiple of 4 floats so 16-byte stores stay aligned
static inline __host__ __device__ int score_stride(int Nk) { return (Nk + 3) & ~3; }

int mask_heads_per_pass(int BH, int G, int Nk) {
  const size_t per = (size_t)G * (size_t)score_stride(Nk) * 4;
  size_t hp = per ? SCORE_STAGE_BUDGET / per : 1;
  if (hp < 1) hp = 1;
  if (hp > (size_t)BH) hp = (size_t)BH;
  return (int)hp;
}

size_t mask_workspace_bytes(int BH, int G, int Nk, int D) {
  const size_t means = align256((size_t)BH * G * D * 2);
  const size_t scores = align256((size_t)mask_heads_per_pass(BH, G, Nk) * G * score_stride(Nk) * 4);
  return 2 * means + scores;
}

// ---------------------------------------------------------------------------------------------
// group mean
// ---------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void k_group_mean(const uint16_t* __restrict__ q, int Nq, int group, int G,
                                                     uint16_t* __restrict__ qhi, uint16_t* __restrict__ qlo) {
  constexpr int NC = D / 8;             // 16-byte chunks per row
  constexpr int RL = 256 / NC;          // row lanes
  __shared__ float part[RL][D + 1];
  const int unit = blockIdx.x;          // bh * G + g
  const int g = unit % G;
  const size_t bh = unit / G;
  const int r0 = g * group;
  const int nrows = min(group, Nq - r0);
  const int chunk = threadIdx.x % NC, rl = threadIdx.x / NC;
  float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const uint16_t* base = q + (bh * Nq + r0) * D + chunk * 8;
  for (int r = rl; r < nrows; r += RL) {
    const u32x4 w = *(const u32x4*)(base + (size_t)r * D);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[2 * e] += bf16_bits_to_float(w[e] & 0xffffu);
      acc[2 * e + 1] += bf16_bits_to_float(w[e] >> 16);
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) part[rl][chunk * 8 + e] = acc[e];
  __syncthreads();
  for (int d = threadIdx.x; d < D; d += 256) {
    float s = 0.0f;
    for (int r = 0; r < RL; ++r) s += part[r][d];
    const float mean = s / (float)nrows;
    const uint32_t hb = pack_bf16x2(mean, 0.0f) & 0xffffu;
    const float rest = mean - bf16_bits_to_float(hb);
    const uint32_t lb = pack_bf16x2(rest, 0.0f) & 0xffffu;
    qhi[(size_t)unit * D + d] = (uint16_t)hb;
    qlo[(size_t)unit * D + d] = (uint16_t)lb;
  }
}

// ---------------------------------------------------------------------------------------------
// scores: one wave = 32 groups x (KT x 32) keys
// ---------------------------------------------------------------------------------------------
constexpr int SC_KT = 4;   // 32-key tiles per wave

template <int D>
__global__ __launch_bounds__(256) void k_scores(const uint16_t* __restrict__ k, const uint16_t* __restrict__ qhi,
                                                 const uint16_t* __restrict__ qlo, int Nk, int G, float scale,
                                                 float* __restrict__ scores, int bh0, int gtiles, int kchunks) {
  constexpr int KSTEPS = D / 16;
  constexpr int RB = D * 2;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int hi = lane >> 5, ql = lane & 31;
  int t = blockIdx.x;
  const int kc = t % kchunks; t /= kchunks;
  const int gt = t % gtiles;
  const int hh = t / gtiles;               // head inside this pass
  const size_t bh = (size_t)bh0 + hh;
  const int g = gt * 32 + ql;

  const __amdgpu_buffer_rsrc_t rh = make_rsrc(qhi + bh * G * D, (uint32_t)G * RB);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(qlo + bh * G * D, (uint32_t)G * RB);
  const uint32_t goff = (uint32_t)(g < G ? g : G) * RB;   // g >= G reads zeros
  bf16x8 bhi[KSTEPS], blo[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    bhi[ks] = __builtin_bit_cast(bf16x8, buffer_load_x4(rh, goff + (2 * ks + hi) * 16));
    blo[ks] = __builtin_bit_cast(bf16x8, buffer_load_x4(rl, goff + (2 * ks + hi) * 16));
  }
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + bh * Nk * D, (uint32_t)Nk * RB);
  float* srow = scores + ((size_t)hh * G + (g < G ? g : 0)) * score_stride(Nk);
  for (int kt = 0; kt < SC_KT; ++kt) {
    const int j0 = ((kc * 4 + wave) * SC_KT + kt) * 32;
    if (j0 >= Nk) break;
    const uint32_t koff = (uint32_t)(j0 + ql) * RB;
    bf16x8 a[KSTEPS];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks)
      a[ks] = __builtin_bit_cast(bf16x8, buffer_load_x4(rk, koff + (2 * ks + hi) * 16));
    f32x16 acc = {};
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ++ks) {
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], bhi[ks], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[ks], blo[ks], acc, 0, 0, 0);
    }
    if (g < G) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int j = j0 + 8 * i + 4 * hi;
        if (j + 3 < Nk) {
          *(f32x4*)(srow + j) = f32x4{acc[4 * i] * scale, acc[4 * i + 1] * scale, acc[4 * i + 2] * scale,
                                      acc[4 * i + 3] * scale};
        } else {
          for (int e = 0; e < 4; ++e)
            if (j + e < Nk) srow[j + e] = acc[4 * i + e] * scale;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------------------
// select + compact
// ---------------------------------------------------------------------------------------------
__device__ inline uint32_t order_key(float s) {
  uint32_t u = __float_as_uint(s == 0.0f ? 0.0f : s);   // -0 and +0 compare equal: one key
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ inline int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  return x;
}

// Exclusive scan of one int per thread over the whole 1024-thread block; returns the block total too.
__device__ inline int block_excl_scan(int x, int* wsum, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_scan(x, lane);
  if (lane == 63) wsum[wave] = incl;
  __syncthreads();
  int before = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < SEL_WAVES; ++w) {
    const int s = wsum[w];
    before += (w < wave) ? s : 0;
    tot += s;
  }
  __syncthreads();
  total = tot;
  return before + incl - x;
}

__device__ inline float block_max(float x, float* red) {
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = red[0];
  for (int w = 1; w < SEL_WAVES; ++w) r = fmaxf(r, red[w]);
  __syncthreads();
  return r;
}

__device__ inline float block_sum(float x, float* red) {
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  float r = 0.0f;
  for (int w = 0; w < SEL_WAVES; ++w) r += red[w];
  __syncthreads();
  return r;
}

__device__ inline int block_min_int(int x, int* red) {
  for (int off = 32; off > 0; off >>= 1) x = min(x, __shfl_xor(x, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = x;
  __syncthreads();
  int r = red[0];
  for (int w = 1; w < SEL_WAVES; ++w) r = min(r, red[w]);
  __syncthreads();
  return r;
}

// Keys of the group's scores: held in VGPRs when NPT > 0 (NPT = keys per thread), otherwise
// re-read from the staged fp32 scores (L2 / MALL resident) in every pass.  Key 0 marks "no key".
template <int NPT>
struct ScoreKeys {
  static constexpr bool IN_REGS = NPT > 0;
  uint32_t u[IN_REGS ? NPT : 1];
  const float* srow;
  int Nk, n;
  __device__ void init(const float* row, int nk) {
    srow = row;
    Nk = nk;
    n = IN_REGS ? NPT : (nk + SEL_THREADS - 1) / SEL_THREADS;
    if (IN_REGS) {
#pragma unroll
      for (int i = 0; i < (IN_REGS ? NPT : 1); ++i) {
        const int j = i * SEL_THREADS + (int)threadIdx.x;
        u[i] = j < Nk ? order_key(srow[j]) : 0u;
      }
    }
  }
  __device__ uint32_t get(int i) const {
    if (IN_REGS) return u[i];
    const int j = i * SEL_THREADS + (int)threadIdx.x;
    return j < Nk ? order_key(srow[j]) : 0u;
  }
};

__device__ inline float key_to_float(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

template <int NPT>
__global__ __launch_bounds__(SEL_THREADS) void k_select(const float* __restrict__ scores, int Nk, int G, int mode,
                                                        int topk, float log_tau, int32_t* __restrict__ idx,
                                                        int32_t* __restrict__ counts, int cap, int bh0) {
  constexpr int MAXROWS = NPT > 0 ? NPT : SATTN_MASK_MAX_NK / SEL_THREADS;
  __shared__ int hist[4096];
  __shared__ int cnt_s[MAXROWS * SEL_WAVES];
  __shared__ int cnt_t[MAXROWS * SEL_WAVES];
  __shared__ int wsum[SEL_WAVES];
  __shared__ float fred[SEL_WAVES];
  __shared__ int ired[SEL_WAVES];
  __shared__ int found[2];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = blockIdx.x / G, g = blockIdx.x % G;
  const size_t unit = ((size_t)bh0 + hh) * G + g;
  ScoreKeys<NPT> sk;
  sk.init(scores + ((size_t)hh * G + g) * score_stride(Nk), Nk);
  const int rows = sk.n;

  uint32_t cut;     // keep u > cut, plus the first `need` keys with u == cut
  int need = 0;
  if (mode == 0) {
    uint32_t prefix = 0, pmask = 0;
    int kk = topk;
    const int shifts[3] = {20, 8, 0};
    const int widths[3] = {12, 12, 8};
    for (int pass = 0; pass < 3; ++pass) {
      const int sh = shifts[pass], nb = 1 << widths[pass];
      for (int b = tid; b < nb; b += SEL_THREADS) hist[b] = 0;
      if (tid == 0) { found[0] = 0; found[1] = 1; }
      __syncthreads();
#pragma unroll(NPT > 0 ? NPT : 1)
      for (int i = 0; i < rows; ++i) {
        const uint32_t u = sk.get(i);
        if ((u & pmask) == prefix && u != 0u) atomicAdd(&hist[(u >> sh) & (nb - 1)], 1);
      }
      __syncthreads();
      // thread t owns bins nb-1-per*t ... (descending); its exclusive scan = count above them
      const int per = nb / SEL_THREADS > 0 ? nb / SEL_THREADS : 1;
      const bool owner = tid * per < nb;
      int local = 0;
      if (owner)
        for (int e = 0; e < per; ++e) local += hist[nb - 1 - (tid * per + e)];
      int total;
      int above = block_excl_scan(local, wsum, total);
      if (owner && above < kk && kk <= above + local) {
        for (int e = 0; e < per; ++e) {
          const int b = nb - 1 - (tid * per + e);
          if (above < kk && kk <= above + hist[b]) {
            found[0] = b;
            found[1] = kk - above;
          }
          above += hist[b];
        }
      }
      __syncthreads();
      prefix |= (uint32_t)found[0] << sh;
      pmask |= (uint32_t)(nb - 1) << sh;
      kk = found[1];
      __syncthreads();
    }
    cut = prefix;
    need = kk;
  } else {
    float m = -INFINITY;
#pragma unroll(NPT > 0 ? NPT : 1)
    for (int i = 0; i < rows; ++i) {
      const uint32_t u = sk.get(i);
      if (u != 0u) m = fmaxf(m, key_to_float(u));
    }
    m = block_max(m, fred);
    float s = 0.0f;
#pragma unroll(NPT > 0 ? NPT : 1)
    for (int i = 0; i < rows; ++i) {
      const uint32_t u = sk.get(i);
      if (u != 0u) s += expf(key_to_float(u) - m);
    }
    s = block_sum(s, fred);
    const float t = m + logf(s) + log_tau;   // log_tau = -inf keeps every key
    // keep s_j >= t  <=>  order_key(s_j) >= order_key(t), i.e. u > cut with cut = key(t) - 1
    const uint32_t kt = (isinf(t) && t < 0.0f) ? 1u : order_key(t);
    cut = kt - 1u;
    need = 0;
  }

  // ---- compaction in ascending key order j = i*1024 + tid ----
#pragma unroll(NPT > 0 ? NPT : 1)
  for (int i = 0; i < rows; ++i) {
    const uint32_t u = sk.get(i);
    const uint64_t bs = __builtin_amdgcn_ballot_w64(u > cut);
    const uint64_t bt = __builtin_amdgcn_ballot_w64(u == cut && need > 0);
    if (lane == 0) {
      cnt_s[i * SEL_WAVES + wave] = __popcll(bs);
      cnt_t[i * SEL_WAVES + wave] = __popcll(bt);
    }
  }
  __syncthreads();
  // exclusive scan over the rows*16 (row, wave) entries in row-major order
  const int nent = rows * SEL_WAVES;
  const int E = (nent + SEL_THREADS - 1) / SEL_THREADS;
  int ls = 0, lt = 0;
  for (int e = 0; e < E; ++e) {
    const int x = tid * E + e;
    if (x < nent) { ls += cnt_s[x]; lt += cnt_t[x]; }
  }
  int tot_s, tot_t;
  const int base_s = block_excl_scan(ls, wsum, tot_s);
  const int base_t = block_excl_scan(lt, wsum, tot_t);
  {
    int rs = base_s, rt = base_t;
    for (int e = 0; e < E; ++e) {
      const int x = tid * E + e;
      if (x < nent) {
        const int a = cnt_s[x], b = cnt_t[x];
        cnt_s[x] = rs; cnt_t[x] = rt;
        rs += a; rt += b;
      }
    }
  }
  __syncthreads();
  int32_t* out = idx + unit * (size_t)cap;
  const int kept = tot_s + min(tot_t, need);
  if (kept > 0) {
#pragma unroll(NPT > 0 ? NPT : 1)
    for (int i = 0; i < rows; ++i) {
      const uint32_t u = sk.get(i);
      const bool st = u > cut;
      const bool tie = u == cut && need > 0;
      const uint64_t bs = __builtin_amdgcn_ballot_w64(st);
      const uint64_t bt = __builtin_amdgcn_ballot_w64(tie);
      const int before_s = cnt_s[i * SEL_WAVES + wave] +
                           (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bs >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bs, 0u));
      const int before_t = cnt_t[i * SEL_WAVES + wave] +
                           (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(bt >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bt, 0u));
      const bool keep = st || (tie && before_t < need);
      const int pos = before_s + min(before_t, need);
      if (keep && pos < cap) out[pos] = i * SEL_THREADS + tid;
    }
    if (tid == 0) counts[unit] = min(kept, cap);
  } else {
    // threshold mode with no key at the cut: keep the arg-max, lowest index on ties
    uint32_t best = 0;
    for (int i = 0; i < rows; ++i) {
      const uint32_t u = sk.get(i);
      best = u > best ? u : best;
    }
    for (int off = 32; off > 0; off >>= 1) {
      const uint32_t o = (uint32_t)__shfl_xor((int)best, off);
      best = o > best ? o : best;
    }
    if (lane == 0) ired[wave] = (int)best;
    __syncthreads();
    uint32_t bmax = 0;
    for (int w = 0; w < SEL_WAVES; ++w) bmax = (uint32_t)ired[w] > bmax ? (uint32_t)ired[w] : bmax;
    __syncthreads();
    int jmin = 0x7fffffff;
    for (int i = 0; i < rows; ++i) {
      const uint32_t u = sk.get(i);
      if (u == bmax && u != 0u) jmin = min(jmin, i * SEL_THREADS + tid);
    }
    jmin = block_min_int(jmin, ired);
    if (tid == 0) {
      out[0] = jmin;
      counts[unit] = 1;
    }
  }
}

template <int D>
static int launch_mask_d(const MaskArgs& a) {
  const int BH = a.B * a.H;
  const int G = (a.Nq + a.group - 1) / a.group;
  hipStream_t st = (hipStream_t)a.stream;
  char* ws = (char*)a.workspace;
  const size_t means = align256((size_t)BH * G * D * 2);
  uint16_t* qhi = (uint16_t*)ws;
  uint16_t* qlo = (uint16_t*)(ws + means);
  float* scores = (float*)(ws + 2 * means);
  hipLaunchKernelGGL((k_group_mean<D>), dim3(BH * G), dim3(256), 0, st, (const uint16_t*)a.q, a.Nq, a.group, G,
                     qhi, qlo);
  int err = (int)hipGetLastError();
  if (err) return err;
  const int hp = mask_heads_per_pass(BH, G, a.Nk);
  const int gtiles = (G + 31) / 32;
  const int kchunks = (a.Nk + 4 * SC_KT * 32 - 1) / (4 * SC_KT * 32);
  const int npt = (a.Nk + SEL_THREADS - 1) / SEL_THREADS;
  const float log_tau = a.mode == 1 ? (a.thresh > 0.0f ? logf(a.thresh) : -INFINITY) : 0.0f;
  for (int bh0 = 0; bh0 < BH; bh0 += hp) {
    const int n = BH - bh0 < hp ? BH - bh0 : hp;
    hipLaunchKernelGGL((k_scores<D>), dim3(n * gtiles * kchunks), dim3(256), 0, st, (const uint16_t*)a.k, qhi, qlo,
                       a.Nk, G, a.scale, scores, bh0, gtiles, kchunks);
#define SATTN_SEL(NPT_)                                                                                   \
  hipLaunchKernelGGL((k_select<NPT_>), dim3(n * G), dim3(SEL_THREADS), 0, st, scores, a.Nk, G, a.mode, a.topk, \
                     log_tau, a.idx, a.counts, a.cap, bh0)
    if (npt <= 4) SATTN_SEL(4);
    else if (npt <= 8) SATTN_SEL(8);
    else if (npt <= 16) SATTN_SEL(16);
    else SATTN_SEL(0);
#undef SATTN_SEL
    err = (int)hipGetLastError();
    if (err) return err;
  }
  return 0;
}

int launch_mask(const MaskArgs& a) { return a.D == 64 ? launch_mask_d<64>(a) : launch_mask_d<128>(a); }

}  // namespace sattn
