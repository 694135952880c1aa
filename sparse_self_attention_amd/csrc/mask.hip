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
//                 of 128 groups x 32 keys so every K row read feeds 128 groups; fp32 scores of a bounded
//                 number of heads are staged in the workspace (up to 2 GB, so one select launch
//                 spans several heads and fills the GPU).
//  k_select       one 1024-thread workgroup per group.  Top-k: the scores kernel also writes every
//                 16th score of a row to a short sample row; the sample's order statistics bracket
//                 the cut to within ~3.5 sigma of sampling error.  One pass over the staged scores
//                 marks the keys above that band and copies the keys inside it to LDS, where a
//                 12 + 12 + 8 bit radix select finds the exact k-th largest (ties go to the lowest
//                 key index).  If the band misses the cut or overflows LDS, the cut is found by
//                 radix passes over the staged scores instead.  Threshold: block max + block sum
//                 of exp, cut = lse + ln(tau), the arg-max key if nothing passes.  Scores are read
//                 with 4-byte loads, 256 consecutive keys per wave and row, 64 per load.  Keep flags
//                 live in plain LDS bitmaps (bit j % 32 of word j / 32) written by wave ballots; the
//                 ascending list comes from popcounts, block scans and mbcnt.
#include <math.h>

#include <atomic>
#include <type_traits>

#include "../../include/sattn.h"
#include "device_common.hpp"
#include "launch.hpp"
#include "stage_layout.hpp"

namespace sattn {

constexpr int SEL_THREADS = 1024;
constexpr int SEL_WAVES = SEL_THREADS / 64;

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
  // the group's rows through a buffer resource (rows past the group read zeros), eight loads in flight
  const __amdgpu_buffer_rsrc_t rq = make_rsrc(q + (bh * Nq + r0) * D, (uint32_t)nrows * D * 2u);
  constexpr int BATCH = 8;
  for (int rb = rl; rb < nrows; rb += BATCH * RL) {
    u32x4 w[BATCH];
#pragma unroll
    for (int k = 0; k < BATCH; ++k) w[k] = buffer_load_x4(rq, (uint32_t)((rb + k * RL) * D + chunk * 8) * 2u);
#pragma unroll
    for (int k = 0; k < BATCH; ++k)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += bf16_bits_to_float(w[k][e] & 0xffffu);
        acc[2 * e + 1] += bf16_bits_to_float(w[k][e] >> 16);
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
constexpr int SC_KT = 16;   // 32-key tiles per workgroup

template <int N>
using IC = std::integral_constant<int, N>;

// S = q_avg K^T: A = 32 group means (rows = groups, hi and lo halves in VGPRs), B = K^T (columns =
// keys).  The 4 waves of a workgroup own 4 different 32-group tiles and walk the same SC_KT x 32
// keys; each 64-key tile is gathered once into LDS with buffer-load-to-LDS (double-buffered, rows
// XOR-swizzled as in the forward) and read by all four waves as two 32-key MFMA tiles (half the
// barriers of 32-key tiles, 2 % faster per mask call).  In the accumulator layout lane l holds
// key j0 + l%32 for 16 groups: each store instruction writes two contiguous 128-byte runs of score
// rows.
template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3, 3))) void k_scores(const uint16_t* __restrict__ k, const uint16_t* __restrict__ qhi,
                                                 const uint16_t* __restrict__ qlo, int Nk, int G, float scale,
                                                 float* __restrict__ scores, float* __restrict__ samples, int bh0,
                                                 int gtiles, int kchunks) {
  constexpr int KSTEPS = D / 16;
  constexpr int RB = D * 2;
  constexpr int NC = D / 8;                       // 16-byte chunks per row
  constexpr int ROWS_PER_LOAD = 1024 / RB;        // rows filled by one 64-lane 16-byte load
  constexpr int TKEYS = 64;                       // keys per LDS tile: two 32-key MFMA tiles
  constexpr int ROWSETS = TKEYS / ROWS_PER_LOAD;
  constexpr int NRS = (ROWSETS + 3) / 4;          // row-sets gathered per wave
  constexpr int TILE = TKEYS * RB;
  constexpr int ROWDIV = 16 / NC;
  // the two stages are LDS objects of their own, so the compiler can tell that the reads of one stage
  // do not depend on the gather in flight into the other one (no wait for it)
  __shared__ __attribute__((aligned(1024))) char kt0[TILE];
  __shared__ __attribute__((aligned(1024))) char kt1[TILE];
  // this workgroup's samples (SC_KT * 32 / SAMPLE_STEP per group), stored as whole runs at the end
  constexpr int SPW = SC_KT * 32 / SAMPLE_STEP;
  __shared__ float ssamp[128 * SPW];
  auto swz = [](int row) { return (row / ROWDIV) % NC; };
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hi = lane >> 5, ql = lane & 31;
  int t = blockIdx.x;
  const int kc = t % kchunks; t /= kchunks;
  const int gq = t % gtiles;               // quad of 32-group tiles
  const int hh = t / gtiles;               // head inside this pass
  const size_t bh = (size_t)bh0 + hh;
  const int gt = gq * 4 + wave;            // this wave's 32-group tile
  const bool active = gt * 32 < G;         // idle waves still take part in the gathers and barriers

  const __amdgpu_buffer_rsrc_t rh = make_rsrc(qhi + bh * G * D, (uint32_t)G * RB);
  const __amdgpu_buffer_rsrc_t rl = make_rsrc(qlo + bh * G * D, (uint32_t)G * RB);
  const int gl = gt * 32 + ql;
  const uint32_t goff = (uint32_t)(gl < G ? gl : G) * RB;   // g >= G reads zeros
  bf16x8 ahi[KSTEPS], alo[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    ahi[ks] = __builtin_bit_cast(bf16x8, buffer_load_x4(rh, goff + (2 * ks + hi) * 16));
    alo[ks] = __builtin_bit_cast(bf16x8, buffer_load_x4(rl, goff + (2 * ks + hi) * 16));
  }
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(k + bh * Nk * D, (uint32_t)Nk * RB);
  uint32_t koff[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) koff[ks] = ql * RB + 16 * ((2 * ks + hi) ^ swz(ql));
  const int row_in = lane / NC, pchunk = lane % NC;
  uint32_t kch[NRS];
#pragma unroll
  for (int j = 0; j < NRS; ++j) kch[j] = 16u * (uint32_t)(pchunk ^ swz((wave + 4 * j) * ROWS_PER_LOAD + row_in));
  const int jbase = kc * SC_KT * 32;
  const int ntile = min(SC_KT * 32 / TKEYS, (Nk - jbase + TKEYS - 1) / TKEYS);
  auto issue = [&](char* kst, int tile) {
#pragma unroll
    for (int j = 0; j < NRS; ++j) {
      const int rs = wave + 4 * j;
      if (ROWSETS % 4 == 0 || rs < ROWSETS) {
        const int p = jbase + tile * TKEYS + rs * ROWS_PER_LOAD + row_in;
        const uint32_t key = (uint32_t)(p < Nk ? p : Nk - 1);
        buffer_load_lds_x4(rk, kst + rs * ROWS_PER_LOAD * RB, key * RB + kch[j]);
      }
    }
  };
  const int stride = score_stride(Nk);
  float* sbase = scores + (size_t)hh * G * stride;
  const int sstride = sample_stride(Nk);
  float* pbase = samples + (size_t)hh * G * sstride;
  const bool sampler = (ql % SAMPLE_STEP) == 0;   // j0 is a multiple of 32, so j % 16 == ql % 16

  // tile t reads stage t % 2 (even tiles stage 0)
  auto body = [&](auto stc, int tile) {
    constexpr int ST = decltype(stc)::value;
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt0();
    __syncthreads();   // tile landed for every wave; the other stage is free again
    if (tile + 1 < ntile) issue(ST == 0 ? kt1 : kt0, tile + 1);
    if (!active) return;
    // the tile's two 32-key halves in turn (rows 32 + r carry the same swizzle as rows r)
#pragma unroll
    for (int sub = 0; sub < TKEYS / 32; ++sub) {
      const char* kt = (ST == 0 ? kt0 : kt1) + sub * 32 * RB;
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < KSTEPS; ++ks) {
        const bf16x8 b = *(const bf16x8*)(kt + koff[ks]);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ahi[ks], b, acc, 0, 0, 0);
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(alo[ks], b, acc, 0, 0, 0);
      }
      const int j = jbase + tile * TKEYS + sub * 32 + ql;
      if (j < Nk) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int g = gt * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
          if (g < G) {
            const float sv = acc[r] * scale;
            sbase[(size_t)g * stride + j] = sv;
            if (sampler) ssamp[(g - gq * 128) * SPW + (j - jbase) / SAMPLE_STEP] = sv;
          }
        }
      }
    }
  };
  issue(kt0, 0);
  int tile = 0;
  for (; tile + 1 < ntile; tile += 2) {
    body(IC<0>{}, tile);
    body(IC<1>{}, tile + 1);
  }
  if (tile < ntile) body(IC<0>{}, tile);
  __syncthreads();   // every wave's samples are in LDS
  const int p0 = jbase / SAMPLE_STEP, plen = sample_len(Nk);
  for (int e = (int)threadIdx.x; e < 128 * SPW; e += 256) {
    const int g = gq * 128 + e / SPW, p = p0 + e % SPW;
    if (g < G && p < plen) pbase[(size_t)g * sstride + p] = ssamp[e];
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

__device__ inline float key_to_float(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

constexpr int SEL_CAND = 4096;                                   // LDS candidates around the cut

// In (digit-)bin search over hist[0..nb): the bin holding the kk-th largest element, counting from
// the top.  Thread t owns bins nb-1-per*t ... (descending); writes found[0] = bin, found[1] = rank
// inside the bin.  Call with every thread of the block.
__device__ inline void find_bin(const int* hist, int nb, int kk, int* wsum, int* found) {
  const int tid = threadIdx.x;
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
}

// Like find_bin for two ranks at once: kA among the counts hA, kB among hB (hA may equal hB).  Each
// distribution holds fewer than 65536 elements, so the two counts travel packed in one int through a
// single block scan.  Writes found[0..1] = (bin, rank inside) for A and found[2..3] for B.
__device__ inline void find_bin_pair(const int* hA, const int* hB, int nb, int kA, int kB, int* wsum, int* found) {
  const int tid = threadIdx.x;
  const int per = nb / SEL_THREADS > 0 ? nb / SEL_THREADS : 1;
  const bool owner = tid * per < nb;
  int local = 0;
  if (owner)
    for (int e = 0; e < per; ++e) {
      const int b = nb - 1 - (tid * per + e);
      local += hA[b] + (hB[b] << 16);
    }
  int total;
  const int above = block_excl_scan(local, wsum, total);
  if (owner) {
    int aA = above & 0xffff, aB = above >> 16;
    for (int e = 0; e < per; ++e) {
      const int b = nb - 1 - (tid * per + e);
      const int cA = hA[b], cB = hB[b];
      if (aA < kA && kA <= aA + cA) { found[0] = b; found[1] = kA - aA; }
      if (aB < kB && kB <= aB + cB) { found[2] = b; found[3] = kB - aB; }
      aA += cA;
      aB += cB;
    }
  }
  __syncthreads();
}

// One 1024-thread workgroup per group.  Keys are visited in rows of SEL_ROW = 4096: wave w covers the 256
// consecutive keys of chunk c = 16 i + w, i.e. keys [256 c, 256 c + 256), and lane l reads keys
// 256 c + 64 e + l (e = 0..3, one 4-byte load each, consecutive across the wave).  A chunk's flags are its
// four wave ballots, one per e: bit l of ballot e flags key 256 c + 64 e + l, so the flag bitmaps are plain
// (bit j % 32 of word j / 32 flags key j) and ballot e of chunk c is words 8c + 2e and 8c + 2e + 1.
//  top-k:     the sample locates a band [key_lo, key_hi] around the cut; one pass (global) marks the
//             keys above it in `strict` and copies the band's keys to LDS; an exact radix select on
//             them resolves the cut; candidates above it join `strict`, ties at the cut go to `tie`.
//             If the band misses the cut or overflows the LDS list, the cut and the flags are
//             computed from global memory instead.
//  threshold: pass 1 max, pass 2 sum of exp, pass 3 marks s >= lse + ln tau in `strict`.
//  Compaction: popcounts of each chunk's bitmap words and block scans give each chunk's base; each kept
//  key writes its index at its rank (mbcnt over the chunk's four ballots).  When every key at the cut is
//  kept (flagged strict) the loop is branch-free; otherwise ties are taken lowest index first up to
//  `need`.
constexpr int SEL_KPT = 4;                          // keys per thread and row (4-byte loads 64 keys apart)
constexpr int SEL_ROW = SEL_KPT * SEL_THREADS;      // keys per row
constexpr int SEL_CHUNK = SEL_KPT * 64;             // keys per (row, wave)
constexpr int SEL_BATCH = 8;                        // rows (four loads each) in flight per thread

static inline size_t select_lds_bytes(int Nk, bool topk) {
  const size_t rows = (size_t)(Nk + SEL_ROW - 1) / SEL_ROW;
  const size_t chunks = rows * SEL_WAVES;
  return 4 * ((topk ? 4096 : 0) + 2 * 8 * chunks + 2 * chunks + (topk ? 2 * SEL_CAND : 0));
}

// Key e (0..3) of thread tid in row i: 256 (16 i + wave) + 64 e + lane.
__device__ inline int sel_key(int i, int tid, int e) { return i * SEL_ROW + (tid >> 6) * SEL_CHUNK + 64 * e + (tid & 63); }

// Score of key e of thread tid in row i (raw bits).  The score row is read through a buffer resource
// (loads past its end return zeros), so the load carries no branch and a batch of them is in flight at once.
__device__ inline uint32_t score_bits(__amdgpu_buffer_rsrc_t rs, int i, int tid, int e) {
  return __builtin_amdgcn_raw_buffer_load_b32(rs, (uint32_t)sel_key(i, tid, e) * 4u, 0, 0);
}

// Order keys of the four keys of thread tid in row i (0 past Nk).
__device__ inline void keys4(__amdgpu_buffer_rsrc_t rs, int i, int tid, int Nk, uint32_t (&u)[SEL_KPT]) {
  uint32_t raw[SEL_KPT];
#pragma unroll
  for (int e = 0; e < SEL_KPT; ++e) raw[e] = score_bits(rs, i, tid, e);
#pragma unroll
  for (int e = 0; e < SEL_KPT; ++e) u[e] = sel_key(i, tid, e) < Nk ? order_key(__uint_as_float(raw[e])) : 0u;
}

// Bitmap word and bit of key j.
__device__ inline int flag_word(int j) { return j >> 5; }
__device__ inline uint32_t flag_bit(int j) { return 1u << (j & 31); }

__device__ inline int mbcnt64(uint64_t b) {
  return (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(b >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)b, 0u));
}

// Lanes 0..7 store the four ballots of chunk c, one word each.
__device__ inline void store_ballots(uint32_t* bits, int c, const uint64_t (&b)[SEL_KPT], int lane) {
  if (lane < 2 * SEL_KPT) {
    const int e = lane >> 1;
    const uint64_t w = e == 0 ? b[0] : e == 1 ? b[1] : e == 2 ? b[2] : b[3];
    bits[8 * c + lane] = (lane & 1) ? (uint32_t)(w >> 32) : (uint32_t)w;
  }
}

// 2 workgroups per CU: at most 64 VGPRs (8 waves per SIMD).
template <bool TOPK>
__global__ __launch_bounds__(SEL_THREADS) __attribute__((amdgpu_waves_per_eu(8, 8)))
void k_select(const float* __restrict__ scores, const float* __restrict__ samples, int Nk, int G, int topk,
                                                        float log_tau, int32_t* __restrict__ idx,
                                                        int32_t* __restrict__ counts, int cap, int bh0) {
  extern __shared__ __attribute__((aligned(16))) int sel_dyn[];   // sized by select_lds_bytes(Nk, TOPK)
  __shared__ int wsum[SEL_WAVES];
  __shared__ float fred[SEL_WAVES];
  __shared__ int ired[SEL_WAVES];
  __shared__ int found[4];
  __shared__ int ncand;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // groups in the reverse of the order the scores kernel wrote them: the last-written rows are still in
  // the last-level cache when the first workgroups read them (4 % faster per mask call than in order)
  const int bid = (int)gridDim.x - 1 - (int)blockIdx.x;
  const int hh = bid / G, g = bid % G;
  const size_t unit = ((size_t)bh0 + hh) * G + g;
  const float* srow = scores + ((size_t)hh * G + g) * score_stride(Nk);
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(srow, (uint32_t)score_stride(Nk) * 4u);
  const int rows = (Nk + SEL_ROW - 1) / SEL_ROW;
  const int chunks = rows * SEL_WAVES;
  const int words = 8 * chunks;
  int* hist = sel_dyn;                                             // 4096 bins (top-k only)
  uint32_t* strict_bits = (uint32_t*)(sel_dyn + (TOPK ? 4096 : 0)); // words
  uint32_t* tie_bits = strict_bits + words;                        // words
  int* cnt_s = (int*)(tie_bits + words);                           // chunks
  int* cnt_t = cnt_s + chunks;                                     // chunks
  uint32_t* cand_key = (uint32_t*)(cnt_t + chunks);                // SEL_CAND (top-k only)
  int* cand_j = (int*)(cand_key + SEL_CAND);                       // SEL_CAND (top-k only)

  for (int w = tid; w < words; w += SEL_THREADS) { strict_bits[w] = 0u; tie_bits[w] = 0u; }
  int need = 0;

  if (TOPK) {
    // ---- 1. the cut's neighbourhood, from the every-16th-key sample of the row ----
    // Keys above key_hi are kept outright; keys in [key_lo, key_hi] become LDS candidates.  The bounds
    // are the sample's order statistics ~3.5 sigma of sampling error either side of the cut's rank,
    // each resolved to 23 of 32 key bits and rounded outwards.  Rows short enough to fit the
    // candidate list skip this: every key is a candidate.
    uint32_t key_hi = 0xffffffffu, key_lo = 1u;
    if (Nk > SEL_CAND) {
      const int S = sample_len(Nk);               // <= 2 * SEL_CAND: cand_key and cand_j are contiguous
      uint32_t* skey = cand_key;
      const float* prow = samples + ((size_t)hh * G + g) * sample_stride(Nk);
      // two 16-byte loads a thread cover up to 8192 samples; both are in flight before either is used
      static_assert(2 * SEL_CAND <= 8 * SEL_THREADS, "two sample quads a thread");
      const __amdgpu_buffer_rsrc_t rp = make_rsrc(prow, (uint32_t)sample_stride(Nk) * 4u);
      f32x4 sq[2];
#pragma unroll
      for (int t = 0; t < 2; ++t)
        sq[t] = __builtin_bit_cast(f32x4, buffer_load_x4(rp, (uint32_t)(tid + t * SEL_THREADS) * 16u));
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int x = 4 * (tid + t * SEL_THREADS) + e;
          if (x < S) skey[x] = order_key(sq[t][e]);
        }
      for (int bb = tid; bb < 4096; bb += SEL_THREADS) hist[bb] = 0;
      __syncthreads();
      const double pk = (double)topk / (double)Nk;
      const int r = (int)ceil(pk * S);
      const int delta = (int)ceil(3.5 * sqrt((double)S * pk * (1.0 - pk))) + 2;
      const bool open_hi = r - delta < 1, open_lo = r + delta > S;
      const int r_hi = open_hi ? 1 : r - delta;
      const int r_lo = open_lo ? S : r + delta;
      for (int x = tid; x < S; x += SEL_THREADS) atomicAdd(&hist[skey[x] >> 20], 1);
      __syncthreads();
      find_bin_pair(hist, hist, 4096, r_hi, r_lo, wsum, found);
      const uint32_t bA = (uint32_t)found[0], bB = (uint32_t)found[2];
      const int kA = found[1], kB = found[3];
      __syncthreads();
      for (int bb = tid; bb < 4096; bb += SEL_THREADS) hist[bb] = 0;
      __syncthreads();
      for (int x = tid; x < S; x += SEL_THREADS) {
        const uint32_t u = skey[x], top = u >> 20, sub = (u >> 9) & 2047u;
        if (top == bA) atomicAdd(&hist[sub], 1);
        if (top == bB) atomicAdd(&hist[2048 + sub], 1);
      }
      __syncthreads();
      find_bin_pair(hist, hist + 2048, 2048, kA, kB, wsum, found);
      if (!open_hi) key_hi = (bA << 20) | ((uint32_t)found[0] << 9) | 0x1ffu;
      if (!open_lo) key_lo = max(1u, (bB << 20) | ((uint32_t)found[2] << 9));
    }
    if (tid == 0) ncand = 0;
    __syncthreads();
    // ---- 2. one pass: keys above the band -> strict bits; keys in it -> LDS candidates ----
    // The pass compares the scores as floats against the band's ends (the order keys' inverse images;
    // an open end is an infinity): order_key is monotone and maps -0 and +0 to one key, as float
    // comparison treats them.  Candidates keep their raw bits and are turned into order keys when the
    // radix select reads them.  (A NaN score is never above or inside the band.)
    // (keys from 0xFF800000 up are +inf and NaNs, keys up to 0x007FFFFF are -inf and NaNs)
    const float hi_f = key_hi >= 0xFF800000u ? INFINITY : key_to_float(key_hi);
    const float lo_f = key_lo <= 0x007FFFFFu ? -INFINITY : key_to_float(key_lo);
    int above_w = 0;   // keys above the band seen by this wave (uniform)
    // Rows go through two buffers of SEL_BATCH / 2 rows: the next buffer's loads are in flight while the
    // current one is sorted, so a workgroup waits about one memory latency for the whole pass.
    constexpr int PB = SEL_BATCH / 2;
    uint32_t sa[PB][SEL_KPT], sb[PB][SEL_KPT];
    auto load_rows = [&](uint32_t (&dst)[PB][SEL_KPT], int i0) {
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int r = 0; r < PB; ++r)
#pragma unroll
        for (int e = 0; e < SEL_KPT; ++e) dst[r][e] = score_bits(rs, i0 + r, tid, e);
      __builtin_amdgcn_sched_barrier(0);
    };
    auto sort_rows = [&](const uint32_t (&sv)[PB][SEL_KPT], int i0) {
#pragma unroll
      for (int r = 0; r < PB; ++r) {
        const int i = i0 + r;
        if (i < rows) {
          uint64_t ab[SEL_KPT], bc[SEL_KPT];
          int nb = 0;
          const int j0 = sel_key(i, tid, 0);
#pragma unroll
          for (int e = 0; e < SEL_KPT; ++e) {
            const float x = __uint_as_float(sv[r][e]);
            const bool valid = j0 + 64 * e < Nk;
            ab[e] = __builtin_amdgcn_ballot_w64(valid && x > hi_f);
            bc[e] = __builtin_amdgcn_ballot_w64(valid && x >= lo_f && x <= hi_f);
            nb += (int)__popcll(bc[e]);
            above_w += (int)__popcll(ab[e]);
          }
          store_ballots(strict_bits, i * SEL_WAVES + wave, ab, lane);
          if (nb > 0) {
            int base = 0;
            if (lane == 0) base = atomicAdd(&ncand, nb);
            base = __builtin_amdgcn_readfirstlane(base);
#pragma unroll
            for (int e = 0; e < SEL_KPT; ++e) {
              if ((bc[e] >> lane) & 1u) {
                const int pos = base + mbcnt64(bc[e]);
                if (pos < SEL_CAND) {
                  cand_key[pos] = sv[r][e];
                  cand_j[pos] = j0 + 64 * e;
                }
              }
              base += (int)__popcll(bc[e]);
            }
          }
        }
      }
    };
    // The loads are unconditional (rows past the end read beyond the buffer resource: zeros, no memory
    // access), so every path reaches a buffer's first use with the same loads outstanding and the waits
    // cover only that buffer.
    load_rows(sa, 0);
    for (int i0 = 0; i0 < rows; i0 += 2 * PB) {
      load_rows(sb, i0 + PB);
      sort_rows(sa, i0);
      load_rows(sa, i0 + 2 * PB);
      sort_rows(sb, i0 + PB);
    }
    if (lane == 0) ired[wave] = above_w;
    __syncthreads();
    int n_above = 0;
    for (int w = 0; w < SEL_WAVES; ++w) n_above += ired[w];
    const int nc = ncand;
    int kk = topk - n_above;
    __syncthreads();
    if (nc <= SEL_CAND && kk >= 1 && kk <= nc) {
      // ---- 3. exact cut among the candidates: radix select in LDS over the low `bits` key bits,
      // the ones that still vary inside [key_lo, key_hi] (the bits above are common to all) ----
      const uint32_t diff = key_lo ^ key_hi;
      int bits = diff ? 32 - __clz(diff) : 0;
      uint32_t prefix = bits == 32 ? 0u : (key_hi >> bits) << bits;
      int ties = nc;   // candidates whose key equals the cut (all of them when the band is one key)
      while (bits > 0) {
        const int w = bits > 12 ? 12 : bits;
        const int sh = bits - w, nb = 1 << w;
        for (int bb = tid; bb < nb; bb += SEL_THREADS) hist[bb] = 0;
        if (tid == 0) { found[0] = 0; found[1] = 1; }
        __syncthreads();
        for (int x = tid; x < nc; x += SEL_THREADS) {
          const uint32_t u = order_key(__uint_as_float(cand_key[x]));
          if (((uint64_t)(u ^ prefix) >> bits) == 0) atomicAdd(&hist[(u >> sh) & (nb - 1)], 1);
        }
        __syncthreads();
        find_bin(hist, nb, kk, wsum, found);
        prefix |= (uint32_t)found[0] << sh;
        kk = found[1];
        ties = hist[found[0]];
        bits = sh;
        __syncthreads();
      }
      need = kk;
      // when every key at the cut is kept they are flagged strict, so only a partial tie uses tie_bits
      const bool all_ties = ties <= need;
      for (int x = tid; x < nc; x += SEL_THREADS) {
        const uint32_t u = order_key(__uint_as_float(cand_key[x]));
        const int jj = cand_j[x];
        if (u > prefix || (all_ties && u == prefix)) atomicOr(&strict_bits[flag_word(jj)], flag_bit(jj));
        else if (u == prefix) atomicOr(&tie_bits[flag_word(jj)], flag_bit(jj));
      }
      __syncthreads();
    } else {
      // ---- fallback: the sampled band missed the cut or overflowed: exact radix over global memory ----
      const int shifts[3] = {20, 8, 0};
      const int widths[3] = {12, 12, 8};
      uint32_t prefix = 0, pmask = 0;
      int ties = 0;
      kk = topk;
      for (int pass = 0; pass < 3; ++pass) {
        const int sh = shifts[pass], nb = 1 << widths[pass];
        for (int bb = tid; bb < nb; bb += SEL_THREADS) hist[bb] = 0;
        if (tid == 0) { found[0] = 0; found[1] = 1; }
        __syncthreads();
        for (int i0 = 0; i0 < rows; i0 += SEL_BATCH) {
          uint32_t u[SEL_BATCH][SEL_KPT];
#pragma unroll
          for (int r = 0; r < SEL_BATCH; ++r) keys4(rs, i0 + r, tid, Nk, u[r]);
#pragma unroll
          for (int r = 0; r < SEL_BATCH; ++r)
#pragma unroll
            for (int e = 0; e < SEL_KPT; ++e)
              if (u[r][e] != 0u && (u[r][e] & pmask) == prefix) atomicAdd(&hist[(u[r][e] >> sh) & (nb - 1)], 1);
        }
        __syncthreads();
        find_bin(hist, nb, kk, wsum, found);
        prefix |= (uint32_t)found[0] << sh;
        pmask |= (uint32_t)(nb - 1) << sh;
        kk = found[1];
        ties = hist[found[0]];   // the last pass resolves every bit: the keys equal to the cut
        __syncthreads();
      }
      need = kk;
      const bool all_ties = ties <= need;
      for (int i = 0; i < rows; ++i) {
        uint32_t u[SEL_KPT];
        keys4(rs, i, tid, Nk, u);
        uint64_t st[SEL_KPT], ti[SEL_KPT];
#pragma unroll
        for (int e = 0; e < SEL_KPT; ++e) {
          st[e] = __builtin_amdgcn_ballot_w64(u[e] > prefix || (all_ties && u[e] == prefix && u[e] != 0u));
          ti[e] = __builtin_amdgcn_ballot_w64(!all_ties && u[e] == prefix && u[e] != 0u);
        }
        store_ballots(strict_bits, i * SEL_WAVES + wave, st, lane);
        store_ballots(tie_bits, i * SEL_WAVES + wave, ti, lane);
      }
      __syncthreads();
    }
  } else {
    __syncthreads();
    float m = -INFINITY;
    for (int i0 = 0; i0 < rows; i0 += SEL_BATCH) {
      uint32_t u[SEL_BATCH][SEL_KPT];
#pragma unroll
      for (int r = 0; r < SEL_BATCH; ++r) keys4(rs, i0 + r, tid, Nk, u[r]);
#pragma unroll
      for (int r = 0; r < SEL_BATCH; ++r)
#pragma unroll
        for (int e = 0; e < SEL_KPT; ++e)
          if (u[r][e] != 0u) m = fmaxf(m, key_to_float(u[r][e]));
    }
    m = block_max(m, fred);
    float ssum = 0.0f;
    for (int i0 = 0; i0 < rows; i0 += SEL_BATCH) {
      uint32_t u[SEL_BATCH][SEL_KPT];
#pragma unroll
      for (int r = 0; r < SEL_BATCH; ++r) keys4(rs, i0 + r, tid, Nk, u[r]);
#pragma unroll
      for (int r = 0; r < SEL_BATCH; ++r)
#pragma unroll
        for (int e = 0; e < SEL_KPT; ++e)
          if (u[r][e] != 0u) ssum += expf(key_to_float(u[r][e]) - m);
    }
    ssum = block_sum(ssum, fred);
    const float t = m + logf(ssum) + log_tau;   // log_tau = -inf keeps every key
    // keep s_j >= t  <=>  order_key(s_j) >= order_key(t), i.e. u > cut with cut = key(t) - 1
    const uint32_t cut = ((isinf(t) && t < 0.0f) ? 1u : order_key(t)) - 1u;
    for (int i0 = 0; i0 < rows; i0 += SEL_BATCH) {
      uint32_t u[SEL_BATCH][SEL_KPT];
#pragma unroll
      for (int r = 0; r < SEL_BATCH; ++r) keys4(rs, i0 + r, tid, Nk, u[r]);
#pragma unroll
      for (int r = 0; r < SEL_BATCH; ++r) {
        if (i0 + r < rows) {
          uint64_t st[SEL_KPT];
#pragma unroll
          for (int e = 0; e < SEL_KPT; ++e) st[e] = __builtin_amdgcn_ballot_w64(u[r][e] > cut);
          store_ballots(strict_bits, (i0 + r) * SEL_WAVES + wave, st, lane);
        }
      }
    }
    __syncthreads();
  }

  // ---- compaction in ascending key order ----
  for (int x = tid; x < chunks; x += SEL_THREADS) {
    int a = 0, b = 0;
#pragma unroll
    for (int k2 = 0; k2 < 8; ++k2) {
      a += __popc(strict_bits[8 * x + k2]);
      b += __popc(tie_bits[8 * x + k2]);
    }
    cnt_s[x] = a;
    cnt_t[x] = b;
  }
  __syncthreads();
  const int E = (chunks + SEL_THREADS - 1) / SEL_THREADS;
  int ls = 0, lt = 0;
  for (int e = 0; e < E; ++e) {
    const int x = tid * E + e;
    if (x < chunks) { ls += cnt_s[x]; lt += cnt_t[x]; }
  }
  int tot_s, tot_t;
  const int base_s = block_excl_scan(ls, wsum, tot_s);
  const int base_t = block_excl_scan(lt, wsum, tot_t);
  {
    int rs = base_s, rt = base_t;
    for (int e = 0; e < E; ++e) {
      const int x = tid * E + e;
      if (x < chunks) {
        const int a = cnt_s[x], b = cnt_t[x];
        cnt_s[x] = rs; cnt_t[x] = rt;
        rs += a; rt += b;
      }
    }
  }
  __syncthreads();
  int32_t* out = idx + unit * (size_t)cap;
  const int kept = tot_s + min(tot_t, need);
  if (kept > 0 && tot_t == 0) {
    // Every key at the cut is kept (the common case: such keys are flagged strict), so a key is listed
    // iff its strict flag is set.  Lane l's keys 4l .. 4l+3 of a chunk land at consecutive positions
    // after the chunk's base and the kept keys of lanes below l.  The stores go through a buffer
    // resource over the list, so an unlisted key (or a position past cap) takes an offset past the end
    // and is dropped: no branches.
    const __amdgpu_buffer_rsrc_t ro = make_rsrc(out, (uint32_t)cap * 4u);
    for (int i = 0; i < rows; ++i) {
      const int x = i * SEL_WAVES + wave;
      const u32x4 s0 = *(const u32x4*)(strict_bits + 8 * x), s1 = *(const u32x4*)(strict_bits + 8 * x + 4);
      const uint32_t w[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
      uint32_t pos = (uint32_t)__builtin_amdgcn_readfirstlane(cnt_s[x]);
      const uint32_t key0 = (uint32_t)(x * SEL_CHUNK + lane);
#pragma unroll
      for (int e = 0; e < SEL_KPT; ++e) {
        // key 256 x + 64 e + l goes after the chunk's kept keys of ballots below e and of lanes below l in
        // ballot e, so the kept keys of one ballot are stored as one contiguous run; an unlisted key's
        // offset has bit 31 set (past the end)
        const uint64_t b = (uint64_t)w[2 * e + 1] << 32 | w[2 * e];
        const uint32_t bit = (uint32_t)(b >> lane) & 1u;
        const uint32_t p = pos + __builtin_amdgcn_mbcnt_hi(w[2 * e + 1], __builtin_amdgcn_mbcnt_lo(w[2 * e], 0u));
        __builtin_amdgcn_raw_buffer_store_b32(key0 + 64u * (uint32_t)e, ro, (p << 2) | ((bit ^ 1u) << 31), 0, 0);
        pos += (uint32_t)__popcll(b);
      }
    }
    if (tid == 0) counts[unit] = min(kept, cap);
  } else if (kept > 0) {
    // only the lowest-index `need` of the keys at the cut are kept
    for (int i = 0; i < rows; ++i) {
      const int x = i * SEL_WAVES + wave;
      uint64_t bs[SEL_KPT], bt[SEL_KPT];
#pragma unroll
      for (int e = 0; e < SEL_KPT; ++e) {
        bs[e] = (uint64_t)strict_bits[8 * x + 2 * e] | ((uint64_t)strict_bits[8 * x + 2 * e + 1] << 32);
        bt[e] = (uint64_t)tie_bits[8 * x + 2 * e] | ((uint64_t)tie_bits[8 * x + 2 * e + 1] << 32);
      }
      // keys of the chunk before key 256 x + 64 e + l: those of ballots below e, then of lanes below l
      int before_s = __builtin_amdgcn_readfirstlane(cnt_s[x]), before_t = __builtin_amdgcn_readfirstlane(cnt_t[x]);
#pragma unroll
      for (int e = 0; e < SEL_KPT; ++e) {
        const int st = (int)((bs[e] >> lane) & 1u), tie = (int)((bt[e] >> lane) & 1u);
        const int ps = before_s + mbcnt64(bs[e]), pt = before_t + mbcnt64(bt[e]);
        const int pos = ps + min(pt, need);
        if ((st || (tie && pt < need)) && pos < cap) out[pos] = x * SEL_CHUNK + 64 * e + lane;
        before_s += (int)__popcll(bs[e]);
        before_t += (int)__popcll(bt[e]);
      }
    }
    if (tid == 0) counts[unit] = min(kept, cap);
  } else {
    // threshold mode with no key at the cut: keep the arg-max, lowest index on ties
    uint32_t best = 0;
    for (int i = 0; i < rows; ++i) {
      uint32_t u[SEL_KPT];
      keys4(rs, i, tid, Nk, u);
#pragma unroll
      for (int e = 0; e < SEL_KPT; ++e) best = u[e] > best ? u[e] : best;
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
      uint32_t u[SEL_KPT];
      keys4(rs, i, tid, Nk, u);
#pragma unroll
      for (int e = 0; e < SEL_KPT; ++e)
        if (u[e] == bmax && u[e] != 0u) jmin = min(jmin, sel_key(i, tid, e));
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
  const int hp = mask_heads_per_pass(BH, G, a.Nk);
  float* samples = (float*)(ws + 2 * means + align256((size_t)hp * G * score_stride(a.Nk) * 4));
  int err = 0;
  log_launch("mask<D=%d> mode %s: %d groups per head, %d of %d heads per pass", D,
             a.mode == 0 ? "top-k" : a.mode == 1 ? "threshold" : "column-sum top-k", G, hp < BH ? hp : BH, BH);
  if (a.mode != 2) {   // the column-sum mode scores from the full queries, not their mean
    hipLaunchKernelGGL((k_group_mean<D>), dim3(BH * G), dim3(256), 0, st, (const uint16_t*)a.q, a.Nq, a.group, G,
                       qhi, qlo);
    err = (int)hipGetLastError();
    if (err) return err;
  }
  const int gtiles = (G + 127) / 128;                       // quads of 32-group tiles
  const int kchunks = (a.Nk + SC_KT * 32 - 1) / (SC_KT * 32);
  const float log_tau = a.mode == 1 ? (a.thresh > 0.0f ? logf(a.thresh) : -INFINITY) : 0.0f;
  // dynamic LDS of the select kernel can exceed 64 KB (86 KB at the largest Nk); the limit is raised once
  // per device (setting it again is harmless, so concurrent first calls need no lock, only atomic flags)
  constexpr int MAX_DEVICES = 64;
  static std::atomic<bool> lds_attr_set[MAX_DEVICES];   // static storage: zero-initialised (false)
  int dev = 0;
  err = (int)hipGetDevice(&dev);
  if (err) return err;
  if (dev < 0 || dev >= MAX_DEVICES || !lds_attr_set[dev].load(std::memory_order_relaxed)) {
    const int max_lds = (int)select_lds_bytes(SATTN_MASK_MAX_NK, true);
    err = (int)hipFuncSetAttribute((const void*)k_select<true>, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    if (!err)
      err = (int)hipFuncSetAttribute((const void*)k_select<false>, hipFuncAttributeMaxDynamicSharedMemorySize, max_lds);
    if (err) return err;
    if (dev >= 0 && dev < MAX_DEVICES) lds_attr_set[dev].store(true, std::memory_order_relaxed);
  }
  for (int bh0 = 0; bh0 < BH; bh0 += hp) {
    const int n = BH - bh0 < hp ? BH - bh0 : hp;
    if (a.mode == 2) {
      ColsumArgs c{a.q, a.k, a.lse, a.Nq, a.Nk, a.D, a.group, a.scale, scores, samples, bh0, n, a.stream};
      err = launch_colsum_scores(c);
      if (err) return err;
    } else {
      hipLaunchKernelGGL((k_scores<D>), dim3(n * gtiles * kchunks), dim3(256), 0, st, (const uint16_t*)a.k, qhi,
                         qlo, a.Nk, G, a.scale, scores, samples, bh0, gtiles, kchunks);
    }
#define SATTN_SEL(T_)                                                                                     \
  hipLaunchKernelGGL((k_select<T_>), dim3(n * G), dim3(SEL_THREADS), select_lds_bytes(a.Nk, T_), st, scores,    \
                     samples, a.Nk, G, a.topk, log_tau, a.idx, a.counts, a.cap, bh0)
    if (a.mode != 1) SATTN_SEL(true);
    else SATTN_SEL(false);
#undef SATTN_SEL
    err = (int)hipGetLastError();
    if (err) return err;
  }
  return 0;
}

int launch_mask(const MaskArgs& a) { return a.D == 64 ? launch_mask_d<64>(a) : launch_mask_d<128>(a); }

}  // namespace sattn
