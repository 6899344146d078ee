// Hypothesis pool ("Decode Before You Hear", page 1, method steps 3 and 5): every draft
// of a session is stored and indexed by its N-grams; after a verify pass the longest
// N-gram of the output's suffix found in the pool gives the continuation to verify next.
//
// Storage: the drafts' tokens one after another (insertion order), and for every stored
// token the end of its draft.  Index: an open-addressing hash table (linear probing)
// from a 64-bit key of (n, the n tokens) to the position right after the most recent
// occurrence of that n-gram that is followed by at least one token of its own draft.
// Positions grow with insertion order, so "most recent" is an atomic maximum and the
// table does not depend on the order in which threads insert.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace sdv {

// splitmix64 finaliser (Steele, Lea, Flood: "Fast splittable pseudorandom number
// generators", OOPSLA 2014)
SDV_DEV unsigned long long mix64(unsigned long long z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// key of the n-gram t[0..n-1]: never 0 (the empty-slot marker)
SDV_DEV unsigned long long ngram_key(const int32_t* t, int n) {
  unsigned long long h = mix64(0x9E3779B97F4A7C15ull * (unsigned long long)(n + 1));
  for (int i = 0; i < n; ++i) h = mix64(h ^ (unsigned long long)(uint32_t)t[i]);
  return h ? h : 1ull;
}

// Append the draft at position count (read once per thread: the insert kernel never
// changes count; the bump kernel after it does).
__global__ __launch_bounds__(256) void pool_store_kernel(PoolArgs a) {
  const int base = *a.count;
  if (base < 0 || base + a.len > a.capacity) {
    if (blockIdx.x == 0 && threadIdx.x == 0) set_err(a.err, 0, POOL_EFULL_STORE);
    return;
  }
  for (int i = blockIdx.x * 256 + threadIdx.x; i < a.len; i += gridDim.x * 256) {
    a.tokens[base + i] = a.draft[i];
    a.seg_end[base + i] = base + a.len;
  }
}

// Index every n-gram (n = 1..max_n) of the draft that is followed by a token of the
// draft: item (end position p, n) covers the n-gram ending at p.
__global__ __launch_bounds__(256) void pool_index_kernel(PoolArgs a) {
  const int base = *a.count;
  if (base < 0 || base + a.len > a.capacity) return;
  const int item = blockIdx.x * 256 + threadIdx.x;
  const int p = item / a.max_n, n = item % a.max_n + 1;
  if (p + 1 >= a.len || p - n + 1 < 0) return;   // needs a following token and n tokens
  const unsigned long long key = ngram_key(a.draft + p - n + 1, n);
  const uint32_t mask = (uint32_t)a.n_slots - 1;
  uint32_t slot = (uint32_t)(key >> 17) & mask;
  for (int probe = 0; probe < a.n_slots; ++probe, slot = (slot + 1) & mask) {
    const unsigned long long prev = atomicCAS(&a.keys[slot], 0ull, key);
    if (prev == 0ull || prev == key) {
      atomicMax(&a.vals[slot], base + p + 1);
      return;
    }
  }
  set_err(a.err, 0, POOL_EFULL_INDEX);
}

__global__ void pool_bump_kernel(PoolArgs a) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    const int base = *a.count;
    if (base >= 0 && base + a.len <= a.capacity) *a.count = base + a.len;
  }
}

hipError_t launch_pool_insert(const PoolArgs& a, hipStream_t s) {
  const int n_store = (a.len + 255) / 256;
  pool_store_kernel<<<n_store, 256, 0, s>>>(a);
  const long long items = (long long)a.len * a.max_n;
  pool_index_kernel<<<(unsigned)((items + 255) / 256), 256, 0, s>>>(a);
  pool_bump_kernel<<<1, 64, 0, s>>>(a);
  return hipGetLastError();
}

// Lookup, one wave per query: lane n-1 (n <= max_n and the suffix length) probes the
// n-gram of the suffix's last n tokens and checks the stored tokens (a different n-gram
// with the same key is no match); the longest match wins, and the wave copies up to
// max_out tokens of its continuation, stopping at the end of that draft.
__global__ __launch_bounds__(64) void pool_lookup_kernel(PoolLookupArgs a) {
  const int q = blockIdx.x;
  const int lane = threadIdx.x;
  const int L = min(max(a.suffix_len[q], 0), a.suffix_cap);
  const int32_t* suf = a.suffix + (size_t)q * a.suffix_cap;
  const int n = lane + 1;
  const int count = *a.count;
  int pos = -1;
  if (n <= a.max_n && n <= L) {
    const unsigned long long key = ngram_key(suf + L - n, n);
    const uint32_t mask = (uint32_t)a.n_slots - 1;
    uint32_t slot = (uint32_t)(key >> 17) & mask;
    for (int probe = 0; probe < a.n_slots; ++probe, slot = (slot + 1) & mask) {
      const unsigned long long k = a.keys[slot];
      if (k == 0ull) break;
      if (k == key) {
        const int p = a.vals[slot];
        bool same = p - n >= 0 && p <= count;
        for (int i = 0; same && i < n; ++i) same = a.tokens[p - n + i] == suf[L - n + i];
        if (same) pos = p;
        break;
      }
    }
  }
  // the longest n with a match
  const unsigned long long found = __ballot(pos >= 0);
  const int best = found ? 63 - __clzll(found) : -1;
  const int p = __shfl(pos, best < 0 ? 0 : best, 64);
  const int end = best < 0 ? 0 : a.seg_end[p];
  const int len = best < 0 ? 0 : min(a.max_out, end - p);
  for (int i = lane; i < a.max_out; i += 64) a.cont[(size_t)q * a.max_out + i] = i < len ? a.tokens[p + i] : -1;
  if (lane == 0) {
    a.cont_len[q] = len;
    if (a.match_n) a.match_n[q] = best + 1;
  }
}

hipError_t launch_pool_lookup(const PoolLookupArgs& a, hipStream_t s) {
  pool_lookup_kernel<<<a.B, 64, 0, s>>>(a);
  return hipGetLastError();
}

// Clear: empty table and storage.
__global__ __launch_bounds__(256) void pool_clear_kernel(PoolArgs a) {
  for (long long i = (long long)blockIdx.x * 256 + threadIdx.x; i < a.n_slots; i += (long long)gridDim.x * 256) {
    a.keys[i] = 0ull;
    a.vals[i] = -1;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) *a.count = 0;
}

hipError_t launch_pool_clear(const PoolArgs& a, hipStream_t s) {
  const long long g = std::min<long long>(4096, (a.n_slots + 255) / 256);
  pool_clear_kernel<<<(unsigned)g, 256, 0, s>>>(a);
  return hipGetLastError();
}

}  // namespace sdv
