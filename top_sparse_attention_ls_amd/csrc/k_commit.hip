// Cache commit (least recently used) and new-token append.
//
// [LeanSparse (arXiv 2611.04671), Abstract]: the indexer-key cache and the
// KV cache are kept apart and reused across generation steps.  [XM-Sparse
// digest, hot buffer section]: a step fetches only the selected rows that
// missed the HBM buffer, and each step's new KV is written back to the full
// history.  The pages give no insertion or eviction policy; the one here is
// least recently used:
//   * an entry of the step (a selected token, or a candidate for the key
//     cache) whose slot-table value lies in [0, n_slots) is a hit, and its
//     slot's stamp becomes `now`;
//   * an entry whose value is negative is a miss; misses are numbered in
//     entry order (ascending position);
//   * the victims are the min(#misses, #slots not hit) slots not hit in this
//     step with the smallest (stamp, slot index), taken in ascending slot
//     order; miss j moves into victim j: the token the victim held loses its
//     slot, and the tables and the stamp are updated.
#include "ls_device.h"
#include "ls_launch.h"

namespace ls {

// One 1024-thread workgroup per request.  The request's stamps sit in LDS
// (one word per slot) with a bitmap of the slots hit in this step; the
// victims' stamp threshold comes from one histogram pass over stamp - min
// when the eligible stamps span fewer than 2048 values (step numbers usually
// do), else from an exact radix select (three digit passes of 11, 11 and 10
// bits over the same 2048-bin LDS histogram); slots of the threshold stamp
// are taken in slot order.  Thread t owns the contiguous slot
// range [t*SE, t*SE + SE) and the entry range [t*EPT, t*EPT + EPT), so
// that prefix sums over threads give slot order and entry order.  Global
// loads are issued all at once per phase (indices clamped, results selected
// afterwards): the table lookups are random reads, and a chain of them per
// thread would serialise their latencies.
//
// Outputs by mode:
//   kCommitDst: dst[b, e] = the entry's slot after the commit, or -1;
//   kCommitHot: for an inserted miss, rows[b, e] := its victim and
//               miss_dst[b, j] := the victim (j = its miss rank; -1 when not
//               inserted) -- the gather then writes the row into the slot;
//   kCommitKey: code[b, e] = the slot of a hit, -(2 + victim) for an
//               inserted miss (the refinement copies the row it reads into
//               that slot), -1 otherwise; n_ins[b] = the number of misses.
//               On entry code[] holds each entry's slot-table value
//               (k_slot_lookup), so the random table reads spread over the
//               grid instead of one workgroup per request.
// For kCommitHot the entries' table values come from rows[] as the top-k
// resolved them (slot tables hold values in [-1, n_slots)).
constexpr int kCommitThreads = 1024;
constexpr int kDigitBins = 2048;

// hist[bin] += 1 for every active lane, with the lanes of the wave that share
// a bin merged into one LDS atomic for up to two distinct bins (stamps are
// step numbers, so a wave's slots usually hold a few values, and one LDS
// address hit by a whole wave's atomics serialises them); lanes left after
// that add their own.
__device__ __forceinline__ void hist_add(uint32_t* hist, uint32_t bin, bool active) {
  const int l = lane_id();
#pragma unroll
  for (int r = 0; r < 2; r++) {
    const uint64_t act = __ballot(active);
    if (act == 0) break;
    const int leader = __ffsll((unsigned long long)act) - 1;
    const uint32_t lb = (uint32_t)__builtin_amdgcn_readlane((int)bin, leader);
    const uint64_t m = __ballot(active && bin == lb);
    if (l == leader) atomicAdd(&hist[lb], (uint32_t)__popcll(m));
    active = active && bin != lb;
  }
  if (active) atomicAdd(&hist[bin], 1u);
}

template <int MODE, int EPT>
__global__ __launch_bounds__(kCommitThreads) void k_cache_commit(
    const int32_t* __restrict__ entries, int n, int32_t* __restrict__ pos2slot,
    int32_t* __restrict__ slot2pos, uint32_t* __restrict__ stamp, int S, int max_ctx,
    uint32_t now_arg, const uint32_t* __restrict__ now_dev, int32_t* __restrict__ out,
    int32_t* __restrict__ rows, int32_t* __restrict__ n_ins) {
  __shared__ uint32_t key[kCommitMaxSlots];        // stamps, then the victim list
  // The key cache (16384 slots per request) keeps each slot's token in LDS
  // and writes its stamps back whole; the hot buffer (a few thousand slots)
  // measured faster with per-slot stamp stores and a read of each victim's
  // token at the end.
  constexpr bool kWholeStamps = MODE == kCommitKey;
  __shared__ int32_t s2p_l[kWholeStamps ? kCommitMaxSlots : 1];  // slot tokens before the commit
  __shared__ uint32_t hitbits[kCommitMaxSlots / 32];
  __shared__ uint32_t hist[kDigitBins];
  __shared__ uint32_t sh_scan[kCommitThreads / kWave];
  __shared__ uint32_t sh_pick[2];
  __shared__ uint32_t sh_lo[kCommitThreads / kWave], sh_hi[kCommitThreads / kWave];

  const int b = blockIdx.x, tid = threadIdx.x;
  // the step's stamp: the argument, or a device counter (graph replays)
  const uint32_t now = now_dev ? *now_dev : now_arg;
  const int32_t* eb = entries + (size_t)b * n;
  int32_t* p2s = pos2slot + (size_t)b * max_ctx;
  int32_t* s2p = slot2pos + (size_t)b * S;
  uint32_t* stb = stamp + (size_t)b * S;
  int32_t* ob = out + (size_t)b * n;

  constexpr int kSlotIters = kCommitMaxSlots / kCommitThreads;
  const int e0 = tid * EPT;
  // the entries and their table values, all loads in flight together
  int32_t t[EPT], sl[EPT];
#pragma unroll
  for (int i = 0; i < EPT; i++) t[i] = eb[min(e0 + i, n - 1)];
  {
    uint32_t sv[kSlotIters];
    int32_t pv[kSlotIters];
#pragma unroll
    for (int i = 0; i < kSlotIters; i++) {
      sv[i] = 0u;
      pv[i] = -1;
      if (kCommitThreads * i < S) {  // uniform: only the rounds that hold slots
        sv[i] = stb[min(tid + kCommitThreads * i, S - 1)];
        if (kWholeStamps) pv[i] = s2p[min(tid + kCommitThreads * i, S - 1)];
      }
    }
#pragma unroll
    for (int i = 0; i < EPT; i++) {
      const bool ok = e0 + i < n && t[i] >= 0 && t[i] < max_ctx;
      t[i] = ok ? t[i] : -1;
      // the entry's table value: looked up here (one workgroup's random
      // reads), or already gathered across the grid and read coalesced: for
      // the hot buffer the top-k's rows (a slot, or hot_slots + rank for a
      // miss), for the key cache the lookup pass's output in code[]
      if (MODE == kCommitHot) {
        const int32_t r = rows[(size_t)b * n + min(e0 + i, n - 1)];
        sl[i] = r < S ? r : -1;
      } else if (MODE == kCommitKey) {
        sl[i] = out[(size_t)b * n + min(e0 + i, n - 1)];
      } else {
        sl[i] = p2s[ok ? t[i] : 0];
      }
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < kSlotIters; i++)
      if (tid + kCommitThreads * i < S) {
        key[tid + kCommitThreads * i] = sv[i];
        if (kWholeStamps) s2p_l[tid + kCommitThreads * i] = pv[i];
      }
  }
  for (int w = tid; w < kCommitMaxSlots / 32; w += kCommitThreads) hitbits[w] = 0u;
  __syncthreads();

  // entries: hits set their slot's bit; misses are flagged (mask over the
  // thread's entries, from the table state before any update)
  uint32_t mmask = 0u, n_m_t = 0u;
#pragma unroll
  for (int i = 0; i < EPT; i++) {
    const int32_t s = t[i] >= 0 ? sl[i] : -1;
    if (s >= 0 && s < S) atomicOr(&hitbits[s >> 5], 1u << (s & 31));
    if (t[i] >= 0 && s < 0) {
      mmask |= 1u << i;
      n_m_t++;
    }
    if ((MODE == kCommitDst || MODE == kCommitKey) && e0 + i < n)
      ob[e0 + i] = (s >= 0 && s < S) ? s : -1;
  }
  __syncthreads();

  // the thread's slots: stamp and whether the step hit it
  const int SE = (S + kCommitThreads - 1) / kCommitThreads;  // <= 16
  const int s0 = tid * SE;
  uint32_t kv[kCommitMaxSlots / kCommitThreads];
  uint32_t elig = 0u, n_hit_t = 0u;
#pragma unroll
  for (int i = 0; i < kCommitMaxSlots / kCommitThreads; i++) {
    const int s = s0 + i;
    kv[i] = 0u;
    if (i < SE && s < S) {
      kv[i] = key[s];
      if ((hitbits[s >> 5] >> (s & 31)) & 1u) n_hit_t++;
      else elig |= 1u << i;
    }
  }
  // misses (low half) and hits (high half) in one scan: each total is at
  // most 16384, so the halves never carry into each other
  uint32_t tot_mh;
  const uint32_t m_base =
      block_excl_scan<kCommitThreads>(n_m_t | (n_hit_t << 16), sh_scan, &tot_mh) & 0xFFFFu;
  const uint32_t n_m = tot_mh & 0xFFFFu, n_h = tot_mh >> 16;
  const uint32_t n_v = min(n_m, (uint32_t)S - n_h);

  // the range of the eligible stamps
  uint32_t lo = 0xFFFFFFFFu, hi = 0u;
#pragma unroll
  for (int i = 0; i < kCommitMaxSlots / kCommitThreads; i++) {
    if ((elig >> i) & 1u) {
      lo = min(lo, kv[i]);
      hi = max(hi, kv[i]);
    }
  }
  lo = (uint32_t)wave_min_u64(lo);
  hi = (uint32_t)wave_max_u64(hi);
  if (lane_id() == 0) {
    sh_lo[wave_id()] = lo;
    sh_hi[wave_id()] = hi;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kCommitThreads / kWave; w++) {
    lo = min(lo, sh_lo[w]);
    hi = max(hi, sh_hi[w]);
  }

  // select T = the n_v-th smallest stamp among the slots not hit, and
  // need = how many slots of stamp T are victims: one histogram pass over
  // stamp - lo when the stamps span fewer than 2048 values (stamps are step
  // numbers, so they usually do), else a radix select over the 32 bits
  uint32_t prefix = 0u, pmask = 0u, need = n_v;
  if (n_v > 0 && hi - lo < (uint32_t)kDigitBins) {
    for (int i = tid; i < kDigitBins; i += kCommitThreads) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kCommitMaxSlots / kCommitThreads; i++)
      hist_add(hist, kv[i] - lo, (elig >> i) & 1u);
    __syncthreads();
    const uint32_t c0 = hist[2 * tid], c1 = hist[2 * tid + 1];
    uint32_t tot;
    const uint32_t base = block_excl_scan<kCommitThreads>(c0 + c1, sh_scan, &tot);
    if (base < need && need <= base + c0) {
      sh_pick[0] = 2u * tid;
      sh_pick[1] = base;
    } else if (base + c0 < need && need <= base + c0 + c1) {
      sh_pick[0] = 2u * tid + 1u;
      sh_pick[1] = base + c0;
    }
    __syncthreads();
    prefix = lo + sh_pick[0];
    need -= sh_pick[1];
  } else if (n_v > 0) {
#pragma unroll 1
    for (int pass = 0; pass < 3; pass++) {
      const int shift = pass == 0 ? 21 : (pass == 1 ? 10 : 0);
      const uint32_t dmask = pass == 2 ? 0x3FFu : 0x7FFu;
      for (int i = tid; i < kDigitBins; i += kCommitThreads) hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int i = 0; i < kCommitMaxSlots / kCommitThreads; i++)
        hist_add(hist, (kv[i] >> shift) & dmask, ((elig >> i) & 1u) && (kv[i] & pmask) == prefix);
      __syncthreads();
      const uint32_t c0 = hist[2 * tid], c1 = hist[2 * tid + 1];
      uint32_t tot;
      const uint32_t base = block_excl_scan<kCommitThreads>(c0 + c1, sh_scan, &tot);
      if (base < need && need <= base + c0) {
        sh_pick[0] = 2u * tid;
        sh_pick[1] = base;
      } else if (base + c0 < need && need <= base + c0 + c1) {
        sh_pick[0] = 2u * tid + 1u;
        sh_pick[1] = base + c0;
      }
      __syncthreads();
      prefix |= sh_pick[0] << shift;
      pmask |= dmask << shift;
      need -= sh_pick[1];
      __syncthreads();  // sh_pick and hist are rewritten by the next pass
    }
  }

  // victims in slot order: stamps below T, then the first `need` slots of
  // stamp T
  uint32_t eq_t = 0u;
#pragma unroll
  for (int i = 0; i < kCommitMaxSlots / kCommitThreads; i++)
    eq_t += (n_v > 0 && ((elig >> i) & 1u) && kv[i] == prefix) ? 1u : 0u;
  uint32_t tot_eq;
  uint32_t eq_rank = block_excl_scan<kCommitThreads>(eq_t, sh_scan, &tot_eq);
  uint32_t vic = 0u, v_t = 0u;
#pragma unroll
  for (int i = 0; i < kCommitMaxSlots / kCommitThreads; i++) {
    if (n_v == 0 || !((elig >> i) & 1u)) continue;
    bool v = kv[i] < prefix;
    if (kv[i] == prefix) {
      v = eq_rank < need;
      eq_rank++;
    }
    if (v) {
      vic |= 1u << i;
      v_t++;
    }
  }
  uint32_t tot_v;
  uint32_t v_rank = block_excl_scan<kCommitThreads>(v_t, sh_scan, &tot_v);
  // misses in entry order move into the victims (tot_v equals n_v; the
  // minimum only keeps every victim read inside the list)
  const uint32_t n_use = min(n_v, tot_v);
  if (kWholeStamps) {
    // new stamps (hit or victim: now) into the LDS copy by each slot's
    // owner, and the token a used victim held loses its slot (cleared by the
    // owner: such a token is cached, so no entry of this step names it)
#pragma unroll
    for (int i = 0; i < kCommitMaxSlots / kCommitThreads; i++) {
      const int s = s0 + i;
      if (i < SE && s < S && (!((elig >> i) & 1u) || ((vic >> i) & 1u))) key[s] = now;
    }
    uint32_t r = v_rank;
#pragma unroll
    for (int i = 0; i < kCommitMaxSlots / kCommitThreads; i++)
      if ((vic >> i) & 1u) {
        const int32_t old = s2p_l[s0 + i];
        if (r < n_use && old >= 0 && old < max_ctx) p2s[old] = -1;
        r++;
      }
    __syncthreads();
    // every stamp written back whole (coalesced)
    for (int s = tid; s < S; s += kCommitThreads) stb[s] = key[s];
  } else {
    // new stamps (hit or victim: now), written by each slot's owner
#pragma unroll
    for (int i = 0; i < kCommitMaxSlots / kCommitThreads; i++) {
      const int s = s0 + i;
      if (i < SE && s < S && (!((elig >> i) & 1u) || ((vic >> i) & 1u))) stb[s] = now;
    }
  }
  __syncthreads();  // then the LDS words are free to hold the victim list
#pragma unroll
  for (int i = 0; i < kCommitMaxSlots / kCommitThreads; i++)
    if ((vic >> i) & 1u) key[v_rank++] = (uint32_t)(s0 + i);
  __syncthreads();

  uint32_t jr[EPT];
  int32_t v[EPT], old[EPT];
  uint32_t j = m_base;
#pragma unroll
  for (int i = 0; i < EPT; i++) {
    const bool m = (mmask >> i) & 1u;
    jr[i] = j;
    v[i] = (m && j < n_use) ? (int32_t)min(key[j], (uint32_t)(S - 1)) : -1;
    j += m ? 1u : 0u;
  }
  // the token each used victim held (key cache: already cleared above)
#pragma unroll
  for (int i = 0; i < EPT; i++) old[i] = kWholeStamps ? -1 : s2p[max(v[i], 0)];
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < EPT; i++) {
    if (!((mmask >> i) & 1u)) continue;
    const int e = e0 + i;
    if (v[i] >= 0) {
      if (old[i] >= 0 && old[i] < max_ctx) p2s[old[i]] = -1;
      p2s[t[i]] = v[i];
      s2p[v[i]] = t[i];
    }
    if (MODE == kCommitDst) ob[e] = v[i];
    if (MODE == kCommitKey) ob[e] = v[i] >= 0 ? -2 - v[i] : -1;
    if (MODE == kCommitHot) {
      ob[jr[i]] = v[i];
      if (v[i] >= 0) rows[(size_t)b * n + e] = v[i];
    }
  }
  // n_ins: misses inserted; for the key cache, the misses (every one of
  // them is read from the key store, inserted or not)
  if (tid == 0 && n_ins) n_ins[b] = (int32_t)(MODE == kCommitKey ? n_m : n_use);
}

// out[b, e] = pos2slot[b, entries[b, e]] (-1 for padding): the table reads
// of the key-cache commit, spread over the grid.
__global__ __launch_bounds__(256) void k_slot_lookup(const int32_t* __restrict__ entries, int n,
                                                     const int32_t* __restrict__ pos2slot,
                                                     int max_ctx, int32_t* __restrict__ out) {
  const int b = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  const int32_t t = entries[(size_t)b * n + e];
  const bool ok = t >= 0 && t < max_ctx;
  const int32_t s = pos2slot[(size_t)b * max_ctx + (ok ? t : 0)];
  out[(size_t)b * n + e] = ok ? s : -1;
}

hipError_t launch_cache_commit(int mode, const int32_t* entries, int n, int32_t* pos2slot,
                               int32_t* slot2pos, uint32_t* stamp, int S, int B, int max_ctx,
                               uint32_t now, const uint32_t* now_dev, int32_t* out,
                               int32_t* rows, int32_t* n_ins, hipStream_t st) {
#define LS_COMMIT_E(M, E)                                                                      \
  hipLaunchKernelGGL((k_cache_commit<M, E>), dim3(B), dim3(kCommitThreads), 0, st, entries, n, \
                     pos2slot, slot2pos, stamp, S, max_ctx, now, now_dev, out, rows, n_ins)
#define LS_COMMIT(M)                                                                          \
  do {                                                                                        \
    if (n <= kCommitThreads) LS_COMMIT_E(M, 1);                                               \
    else if (n <= 2 * kCommitThreads) LS_COMMIT_E(M, 2);                                      \
    else if (n <= 4 * kCommitThreads) LS_COMMIT_E(M, 4);                                      \
    else if (n <= 8 * kCommitThreads) LS_COMMIT_E(M, 8);                                      \
    else LS_COMMIT_E(M, 16);                                                                  \
  } while (0)
  if (mode == kCommitKey) {
    hipLaunchKernelGGL(k_slot_lookup, dim3((n + 255) / 256, B), dim3(256), 0, st, entries, n,
                       pos2slot, max_ctx, out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (mode == kCommitHot) LS_COMMIT(kCommitHot);
  else if (mode == kCommitKey) LS_COMMIT(kCommitKey);
  else LS_COMMIT(kCommitDst);
#undef LS_COMMIT
#undef LS_COMMIT_E
  return hipGetLastError();
}

// ------------------------------------------------------------- append ----
// The step's new token of request b goes to position ctx_len[b] (when it is
// below max_ctx): its int8 key into k8, its compact key into kc, its KV row
// into the pool; then ctx_len[b] grows by one.  One wave per request; every
// lane reads ctx_len before lane 0 writes it (one load instruction for the
// wave, and lane 0's store depends on its own loaded value).
__global__ __launch_bounds__(64) void k_append_token(const int8_t* __restrict__ new_k8,
                                                     const uint4* __restrict__ new_kv,
                                                     int8_t* k8, uint8_t* __restrict__ kc,
                                                     uint4* pool, int32_t* ctx_len, int D,
                                                     int max_ctx, int row_chunks) {
  const int b = blockIdx.x, l = threadIdx.x;
  const int32_t p = ctx_len[b];
  if (p < 0 || p >= max_ctx) return;
  const size_t tok = (size_t)b * max_ctx + p;
  // key: lane l < D/16 copies 16 bytes and packs them into 8 compact bytes
  if (l < D / 16) {
    const uint4 x = *(const uint4*)(new_k8 + (size_t)b * D + 16 * l);
    *(uint4*)(k8 + tok * D + 16 * l) = x;
    const uint32_t w4[4] = {x.x, x.y, x.z, x.w};
    uint32_t packed[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 4; i++) {
      uint32_t two = 0u;
#pragma unroll
      for (int k = 0; k < 4; k++) {
        const int32_t e = (int32_t)(int8_t)((w4[i] >> (8 * k)) & 0xFFu) >> 4;
        two |= ((uint32_t)e & 15u) << (4 * k);
      }
      packed[i >> 1] |= two << (16 * (i & 1));
    }
    *(uint2*)(kc + tok * (D / 2) + 8 * l) = make_uint2(packed[0], packed[1]);
  }
  if (pool) {
    for (int c = l; c < row_chunks; c += 64)
      pool[tok * row_chunks + c] = new_kv[(size_t)b * row_chunks + c];
  }
  if (l == 0) ctx_len[b] = p + 1;
}

hipError_t launch_append_token(const int8_t* new_k8, const void* new_kv, int8_t* k8,
                               uint8_t* kc, void* pool, int32_t* ctx_len, int B, int D,
                               int max_ctx, int row_elems, hipStream_t st) {
  hipLaunchKernelGGL(k_append_token, dim3(B), dim3(64), 0, st, new_k8, (const uint4*)new_kv, k8,
                     kc, (uint4*)pool, ctx_len, D, max_ctx, row_elems * 2 / 16);
  return hipGetLastError();
}

}  // namespace ls
