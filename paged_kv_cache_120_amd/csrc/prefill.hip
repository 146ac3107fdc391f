// Chunked prefill over the paged cache for gfx950: the attention of many
// query rows per sequence (a prompt chunk) over that sequence's keys,
// reached through its block table.  [BOOK] §4.5 (2): the backend takes the
// query tokens of every request delimited by cu_seqlens_q, the keys per
// request and the block table; §4.5 (1): the chunk's K/V are in the cache
// before it is read.  Row j of a T-row chunk sits at position n - T + j and
// attends to keys 0 .. n - T + j (causal).
//
// Where the decode kernels stream each key once per query column tile,
// here the rows x heads that share a kv head are the columns of matrix-core
// products, 128 per workgroup (32 per wave), so each key tile is read from
// HBM once per 128 rows and from LDS once per 32:
//  - a workgroup (kv head, row tile, sequence) walks the keys its rows can
//    see in tiles of 64, staged through LDS (K and V rows as stored,
//    padded), the next tile's global loads in flight while the current one
//    is computed, block addressing scalar;
//  - scores S^T = K Q^T per 16-key block with 16x16x32 MFMAs (keys on the
//    A rows, the wave's 16-row query blocks on the B columns, Q in
//    registers for the whole walk; four key blocks in flight), the causal
//    mask only on tiles that reach past a wave's first row;
//  - the online softmax of [BOOK] §4.6 per query row (each row's maximum
//    and sum reduced over its four lane groups with permlane swaps)
//    against a lazy reference, as in the decode kernels: the accumulators
//    are rescaled only when a tile's maximum passes the reference by more
//    than 2^8 (weights stay <= 2^8 before the fp16 rounding of the
//    product), and O / L cancels the reference at the end;
//  - O^T += V^T P^T with 16x16x16 MFMAs, each V^T fragment one transposing
//    LDS read (gfx950's ds_read_b64_tr_b16) of the row-major tile, and P^T
//    taken from the score layout as it is.
// Measured on MI355X (512-token chunks, GQA-4): longest work first 12%
// faster than grid order (16 sequences of U[512, 4096]); transposing reads 12%
// faster than four 16-bit reads per fragment, 64-key tiles 2.5% faster
// than 32, scalar block addressing with the mask on edge tiles only 21%
// faster than per-lane addressing and masking, the lazy reference 5%
// faster than the exact running maximum.  Slower and not kept: V stored as
// interleaved key pairs or transposed by scatter stores, two LDS buffers
// with one barrier per tile, 8 waves of 16 rows.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "common.h"
#include "prefill.h"

namespace pa {
namespace {

constexpr int kPfWaves = 4;
constexpr int kPfThreads = 64 * kPfWaves;
constexpr int kWaveRows = kPrefillRows / kPfWaves;   // 32: two 16-row blocks
constexpr int kKeyTile = 64;                         // four 16-key blocks
constexpr int KB = kKeyTile / 16;
constexpr float kPfLog2e = 1.4426950408889634f;
constexpr float kPfLn2 = 0.6931471805599453f;

constexpr float kPfSlack = 8.f;      // reference slack, base-2 units

// K and V rows as stored.  K rows padded by 8 halves (the 16 rows of a
// fragment read land 4 banks apart); V rows by 16 (a transposing read takes
// 4 rows x 32 bytes per lane group: rows 8 banks apart, groups 32)
template <int D>
struct PrefillSmem {
  _Float16 k[kKeyTile][D + 8];
  _Float16 v[kKeyTile][D + 16];
};

typedef short s16x4 __attribute__((ext_vector_type(4)));

// Values of lane l and lane l ^ 16 (l ^ 32): gfx950's permlane swaps with
// both operands x leave the pair {x[l], x[l ^ 16]} in the two results, in
// a lane-dependent order, so a max or a sum of the two is the xor
// reduction without a round trip through LDS
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x),
                                                  false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D, int B, int G, bool SPLIT>
__global__ __launch_bounds__(kPfThreads) __attribute__((amdgpu_waves_per_eu(D == 128 ? 2 : 3)))
void prefill_kernel(PrefillArgs a) {
  constexpr int KS = D / 32;            // 32-channel k-steps of the score MFMA
  constexpr int DB = D / 16;            // 16-channel blocks of the output
  constexpr int CPR = D / 8;            // 16-byte chunks per key row
  constexpr int U = kKeyTile * CPR / kPfThreads;   // chunks per thread per tile
  static_assert(U * kPfThreads == kKeyTile * CPR, "tile chunks split evenly");
  __shared__ PrefillSmem<D> sm;

  const int kvh = blockIdx.x;
  // longest work first (the dispatcher hands out workgroups in grid order):
  // grid.z index z takes the sequence with the z-th largest context (ties
  // by index; batches of up to 256 sequences, larger ones in batch order),
  // and its row tiles go last to first (later rows see more keys)
  int s = blockIdx.z;
  int part = 0;
  const int S = gridDim.z;
  if constexpr (SPLIT) {           // z = partition * num_seqs + sequence
    part = blockIdx.z / a.num_seqs;
    s = blockIdx.z % a.num_seqs;
  } else if (S <= kPfThreads) {
    __shared__ int lens[kPfThreads];
    __shared__ int pick;
    const int c = (int)threadIdx.x;
    const int nc = c < S ? a.context_lens[c] : 0;
    lens[c] = nc;
    __syncthreads();
    if (c < S) {
      int rank = 0;
      for (int t = 0; t < S; ++t) {
        const int nt = lens[t];
        rank += (nt > nc) || (nt == nc && t < c);
      }
      if (rank == (int)blockIdx.z) pick = c;
    }
    __syncthreads();
    s = pick;
  }
  const int q0 = a.cu_seqlens_q[s];
  const int T = a.cu_seqlens_q[s + 1] - q0;
  const int rows = T * G;
  const int r0 = (gridDim.y - 1 - blockIdx.y) * kPrefillRows;
  if (T <= 0 || r0 >= rows) return;
  const int H = a.num_heads;
  const int Hkv = a.num_kv_heads;
  const int max_tok = a.max_blocks_per_seq * B;
  int n = a.context_lens[s];
  n = n < max_tok ? n : max_tok;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;
  const int grp = lane >> 4;

  // keys any row of the workgroup sees: 0 .. n - T + last token; in the
  // split mode the partition's keys [k0, kend) of them (none: no states,
  // the reduce reads only partitions that hold keys of a row)
  const int rl = (r0 + kPrefillRows < rows ? r0 + kPrefillRows : rows) - 1;
  int kend = n > 0 ? n - T + rl / G + 1 : 0;
  const int k0 = SPLIT ? part * a.partition_size : 0;
  if constexpr (SPLIT) {
    kend = kend < k0 + a.partition_size ? kend : k0 + a.partition_size;
    if (kend <= k0) return;
  }

  // this lane's two B columns: query rows r = r0 + wave*32 + rb*16 + col,
  // token r / G and head r % G of the chunk; key limit p (none below 0)
  int prow[2];
  int orow[2];                 // element offsets (< 2^31: checked by the host)
  f16x8 qf[2][KS];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    const int r = r0 + wave * kWaveRows + rb * 16 + col;
    const int j = r / G;
    const bool ok = r < rows && q0 + j < a.num_q_tokens;
    prow[rb] = ok && n > 0 ? n - T + j : -1;    // no keys: the row gets zeros
    orow[rb] = ok ? ((q0 + j) * H + kvh * G + r % G) * D : -1;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 v = {0u, 0u, 0u, 0u};
      if (ok) v = *reinterpret_cast<const u32x4*>(a.query + orow[rb] + ks * 32 + grp * 8);
      qf[rb][ks] = __builtin_bit_cast(f16x8, v);
    }
  }
  if constexpr (SPLIT) {
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) prow[rb] = prow[rb] < kend - 1 ? prow[rb] : kend - 1;
  }

  // the wave's first row sees the fewest keys: tiles within them need no
  // causal mask (wave-uniform)
  const int rw = r0 + wave * kWaveRows;
  int pfirst = rw < rows && n > 0 ? n - T + rw / G : -1;
  if constexpr (SPLIT) pfirst = pfirst < kend - 1 ? pfirst : kend - 1;

  // Chunk u of a lane: key kw(u) + lane / CPR of the tile, channels
  // (lane % CPR) * 8 .. +7 of head kvh.  A wave's chunk u covers 64 / CPR
  // consecutive keys, aligned to that count, so they lie in one block
  // (B >= 16): the table entry, the block base and the record limit are
  // scalar, and a lane adds a 32-bit offset.  Keys past kend, or a block id
  // outside the pool, read as zeros (buffer record limit).
  const int* bt = a.block_tables + (size_t)s * a.max_blocks_per_seq;
  const uint32_t row_bytes = (uint32_t)Hkv * D * 2;
  const uint64_t blk_bytes = (uint64_t)B * row_bytes;
  const char* kbase = a.key_cache + (size_t)kvh * D * 2;
  const char* vbase = a.value_cache + (size_t)kvh * D * 2;
  const uint32_t lane_off = (uint32_t)(lane / CPR) * row_bytes + (lane % CPR) * 16;
  u32x4 kr[U], vr[U];
  auto fetch = [&](int kt0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int kw = __builtin_amdgcn_readfirstlane((64 * wave + kPfThreads * u) / CPR);
      const int tw = kt0 + kw;
      const int lb = tw / B;
      const int blk = tw < kend ? bt[lb] : -1;
      int valid = kend - lb * B;
      valid = valid < B ? valid : B;
      const bool ok = tw < kend && (unsigned)blk < (unsigned)a.num_blocks;
      const uint32_t nrec = ok ? (uint32_t)valid * row_bytes : 0u;
      const uint64_t boff = ok ? (uint64_t)blk * blk_bytes : 0;
      const uint32_t voff = (uint32_t)(tw % B) * row_bytes + lane_off;
      kr[u] = load16<0>(make_rsrc(kbase + boff, nrec), voff);
      vr[u] = load16<0>(make_rsrc(vbase + boff, nrec), voff);
    }
  };

  const float sl2 = a.scale * kPfLog2e;
  float m[2] = {-INFINITY, -INFINITY};
  float l[2] = {0.f, 0.f};
  f32x4 o[2][DB];
#pragma unroll
  for (int rb = 0; rb < 2; ++rb)
#pragma unroll
    for (int db = 0; db < DB; ++db) o[rb][db] = (f32x4){0.f, 0.f, 0.f, 0.f};

  if (kend > k0) fetch(k0);
  for (int kt0 = k0; kt0 < kend; kt0 += kKeyTile) {
    __syncthreads();                     // every wave is done with the last tile
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int c = (int)threadIdx.x + u * kPfThreads;
      const int kk = c / CPR;
      *reinterpret_cast<u32x4*>(&sm.k[kk][(c % CPR) * 8]) = kr[u];
      *reinterpret_cast<u32x4*>(&sm.v[kk][(c % CPR) * 8]) = vr[u];
    }
    __syncthreads();
    if (kt0 + kKeyTile < kend) fetch(kt0 + kKeyTile);

    // S^T: A rows = keys kb*16 + col, B columns = query rows; lane keeps
    // keys kt0 + kb*16 + 4*grp + i of its two rows (raw dot products)
    float sc[KB][2][4];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f16x8 kf[KS];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        kf[ks] = *reinterpret_cast<const f16x8*>(&sm.k[kb * 16 + col][ks * 32 + grp * 8]);
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(kf[ks], qf[rb][ks], acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[kb][rb][i] = acc[i];
      }
    }
    if (kt0 + kKeyTile - 1 > pfirst) {          // a tile on the causal edge
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kt0 + kb * 16 + grp * 4 + i > prow[rb]) sc[kb][rb][i] = -INFINITY;
    }
    // online softmax of each row (its keys spread over the 4 lane groups),
    // in base-2 units against the lazy reference m
#pragma unroll
    for (int rb = 0; rb < 2; ++rb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, sc[kb][rb][i]);
      mx = max_xor32(max_xor16(mx));
      mx *= sl2;
      if (__builtin_amdgcn_ballot_w64(mx > m[rb] + kPfSlack)) {
        const float mn = fmaxf(m[rb], mx);
        const float al = fast_exp2(m[rb] - (mn == -INFINITY ? 0.f : mn));
        l[rb] *= al;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[rb][db] *= al;
        m[rb] = mn;
      }
      const float sh = m[rb] == -INFINITY ? 0.f : m[rb];
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sc[kb][rb][i] = fast_exp2(__builtin_fmaf(sc[kb][rb][i], sl2, -sh));
          l[rb] += sc[kb][rb][i];
        }
    }
    // O^T += V^T P^T: A = V^T (channel db*16 + col, keys 4*grp + 0..3 of
    // block kb), B = P^T as the score layout holds it
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      f16x4 pb[2];
#pragma unroll
      for (int rb = 0; rb < 2; ++rb)
#pragma unroll
        for (int i = 0; i < 4; ++i) pb[rb][i] = (_Float16)sc[kb][rb][i];
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        // ds_read_b64_tr_b16: within each 16-lane group, lane j receives
        // element j % 4 of the 8-byte rows that lanes 4e + j / 4 address
        // (e = 0..3); lane s of group grp addresses channels
        // db*16 + 4*(s%4) .. +3 of key kb*16 + 4*grp + s/4, so lane col gets
        // channel db*16 + col of keys 4*grp + 0..3: the A fragment
        const f16x4 va = __builtin_bit_cast(f16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)&sm.v[kb * 16 + grp * 4 + col / 4]
                                                             [db * 16 + 4 * (col % 4)]));
#pragma unroll
        for (int rb = 0; rb < 2; ++rb)
          o[rb][db] = __builtin_amdgcn_mfma_f32_16x16x16f16(va, pb[rb], o[rb][db], 0, 0, 0);
      }
    }
  }

  // rows: the sum over the 4 lane groups, then O / L (zeros without keys);
  // lane holds channels db*16 + 4*grp .. +3 of its rows
#pragma unroll
  for (int rb = 0; rb < 2; ++rb) {
    float L = l[rb];
    L = sum_xor32(sum_xor16(L));
    if (orow[rb] < 0) continue;
    if constexpr (SPLIT) {
      // the partition's state of rows that see one of its keys
      if (prow[rb] < k0) continue;
      const size_t pi = (size_t)(orow[rb] / D) * a.max_partitions + part;
      if (grp == 0) {
        a.ws_max[pi] = m[rb] * kPfLn2;
        a.ws_sum[pi] = L;
      }
#pragma unroll
      for (int db = 0; db < DB; ++db)
        *reinterpret_cast<f32x4*>(a.ws_out + pi * D + db * 16 + grp * 4) = o[rb][db];
      continue;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      f16x4 h;
#pragma unroll
      for (int i = 0; i < 4; ++i) h[i] = (_Float16)(o[rb][db][i] * inv);
      *reinterpret_cast<f16x4*>(a.out + orow[rb] + db * 16 + grp * 4) = h;
    }
  }
}

// The fold: D/16 lanes per (row, head), each lane 16 channels, so a wave
// holds 1024/D rows x heads and their load chains overlap.  The row's
// partitions 0 .. pos / partition_size are folded with the [BOOK] §4.6
// recurrence: the max of their m, then L and O scaled by exp(m_p - max)
// and summed in partition order (bitwise repeatable; every lane of a row
// takes the same sums).  Partitions go four at a time, their scalars and
// rows loaded together.  A row before the first key, or of a sequence
// without keys, gets zeros.
template <int D>
__global__ __launch_bounds__(256) void prefill_fold_kernel(PrefillArgs a) {
  constexpr int CH = 16;                        // channels per lane
  constexpr int NV = CH / 4;
  constexpr int LPI = D / CH;                   // lanes per (row, head)
  constexpr int IPW = 64 / LPI;
  constexpr int K = 4;                          // partitions per step
  const int H = a.num_heads;
  const int lane = threadIdx.x & 63;
  const int li = lane % LPI;
  const int64_t item = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * IPW + lane / LPI;
  if (item >= (int64_t)a.num_q_tokens * H) return;   // uniform per row x head
  const int r = (int)(item / H);
  int lo = 0, hi = a.num_seqs - 1;              // sequence holding row r
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.cu_seqlens_q[mid] <= r) lo = mid;
    else hi = mid - 1;
  }
  const int T = a.cu_seqlens_q[lo + 1] - a.cu_seqlens_q[lo];
  int n = a.context_lens[lo];
  n = n < a.max_tokens ? n : a.max_tokens;
  const int pos = n - T + (r - a.cu_seqlens_q[lo]);
  _Float16* o = a.out + item * D + li * CH;
  if (n <= 0 || pos < 0) {
#pragma unroll
    for (int i = 0; i < CH / 8; ++i) reinterpret_cast<u32x4*>(o)[i] = (u32x4){0u, 0u, 0u, 0u};
    return;
  }
  int np = pos / a.partition_size + 1;
  np = np < a.max_partitions ? np : a.max_partitions;
  const size_t base = (size_t)item * a.max_partitions;
  const float* wo = a.ws_out + base * D + li * CH;

  float m[K], l[K];
  f32x4 v[K][NV];
  auto load = [&](int c) {
#pragma unroll
    for (int u = 0; u < K; ++u) {
      const bool in = c + u < np;
      m[u] = in ? a.ws_max[base + c + u] : -INFINITY;
      l[u] = in ? a.ws_sum[base + c + u] : 0.f;
#pragma unroll
      for (int e = 0; e < NV; ++e)
        v[u][e] = in ? *reinterpret_cast<const f32x4*>(wo + (size_t)(c + u) * D + 4 * e)
                     : (f32x4){0.f, 0.f, 0.f, 0.f};
    }
  };
  load(0);                                      // the first step in flight
  float mx = -INFINITY;
#pragma unroll
  for (int u = 0; u < K; ++u) mx = fmaxf(mx, m[u]);
  for (int c = K; c < np; c += K) {
#pragma unroll
    for (int u = 0; u < K; ++u) if (c + u < np) mx = fmaxf(mx, a.ws_max[base + c + u]);
  }
  float S = 0.f;
  f32x4 acc[NV];
#pragma unroll
  for (int e = 0; e < NV; ++e) acc[e] = (f32x4){0.f, 0.f, 0.f, 0.f};
  for (int c = 0; c < np; c += K) {
    if (c > 0) load(c);
#pragma unroll
    for (int u = 0; u < K; ++u) {
      if (c + u >= np) break;
      const float f = fast_exp2((m[u] - mx) * kPfLog2e);
      S += l[u] * f;
#pragma unroll
      for (int e = 0; e < NV; ++e) acc[e] += v[u][e] * f;
    }
  }
#pragma unroll
  for (int e = 0; e < NV; e += 2) {
    f16x8 h;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      h[i] = (_Float16)(acc[e][i] / S);
      h[4 + i] = (_Float16)(acc[e + 1][i] / S);
    }
    reinterpret_cast<u32x4*>(o)[e / 2] = __builtin_bit_cast(u32x4, h);
  }
}

template <int D, int B, bool SP>
hipError_t launch_dbs(const PrefillArgs& a, int G, dim3 grid, hipStream_t st) {
  switch (G) {
    case 1: hipLaunchKernelGGL((prefill_kernel<D, B, 1, SP>),
                               grid, dim3(kPfThreads), 0, st, a); break;
    case 2: hipLaunchKernelGGL((prefill_kernel<D, B, 2, SP>),
                               grid, dim3(kPfThreads), 0, st, a); break;
    case 4: hipLaunchKernelGGL((prefill_kernel<D, B, 4, SP>),
                               grid, dim3(kPfThreads), 0, st, a); break;
    case 8: hipLaunchKernelGGL((prefill_kernel<D, B, 8, SP>),
                               grid, dim3(kPfThreads), 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const PrefillArgs& a, int B, int G, dim3 grid, bool split,
                    hipStream_t st) {
  switch (B) {
    case 16: return split ? launch_dbs<D, 16, true>(a, G, grid, st)
                          : launch_dbs<D, 16, false>(a, G, grid, st);
    case 32: return split ? launch_dbs<D, 32, true>(a, G, grid, st)
                          : launch_dbs<D, 32, false>(a, G, grid, st);
    case 64: return split ? launch_dbs<D, 64, true>(a, G, grid, st)
                          : launch_dbs<D, 64, false>(a, G, grid, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill_fold(const PrefillArgs& a, int head_size,
                               hipStream_t stream) {
  const int64_t items = (int64_t)a.num_q_tokens * a.num_heads;
  if (items <= 0) return hipSuccess;
  const int64_t per_wg = 4 * (64 / (head_size / 16));  // rows x heads per workgroup
  const dim3 grid((unsigned)((items + per_wg - 1) / per_wg));
  switch (head_size) {
    case 64: hipLaunchKernelGGL((prefill_fold_kernel<64>), grid, dim3(256), 0, stream, a); break;
    case 128: hipLaunchKernelGGL((prefill_fold_kernel<128>), grid, dim3(256), 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_prefill(const PrefillArgs& a, int head_size, int block_size,
                          int group, dim3 grid, bool split, hipStream_t stream) {
  switch (head_size) {
    case 64: return launch_d<64>(a, block_size, group, grid, split, stream);
    case 128: return launch_d<128>(a, block_size, group, grid, split, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
