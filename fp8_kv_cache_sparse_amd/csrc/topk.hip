// Top-k position selection on gfx950 (vLLM blog "DeepSeek-V4.1-Flash sur vLLM",
// sections TL;DR and "Kernels": the DeepSelect top-k over the indexer scores).
//
// Order: score descending, ties to the lower position.  Every candidate is given
// the 64-bit composite c = (key(score) << 32) | (0xFFFFFFFF - position), where
// key() is the order-preserving float->uint32 map; composites are unique, so the
// k largest composites are exactly the wanted set and the selection is a radix
// select on c (11-bit digits, most significant first).
//
// Short rows (<= kSmallN columns): one 1024-thread workgroup per query keeps the
// keys in LDS and runs the whole select there.
// Long rows: (1) many workgroups per query build a 4096-bin histogram of the top
// 12 key bits; the last one to finish finds the bin d1 holding the k-th entry;
// (2) many workgroups per query copy every entry above d1 to the output set and
// every entry in d1 to a candidate buffer; (3) one workgroup per query finishes
// the select inside d1 from LDS (or, if d1 is too full, by re-reading the row),
// sorts the k positions and writes them.
#include "common.h"

namespace smqa {

constexpr int kSmallN = 16384;
constexpr int kChunk = 4096;
constexpr int kCap = 12288;          // candidate-buffer capacity per query (entries of bin d1)
constexpr int kHistBins = 4096;

struct TopkState {
  int d1;        // threshold bin of the top 12 key bits; -1: every valid entry is selected
  int above;     // entries in bins > d1 (all selected)
  int cnt1;      // entries in bin d1
  int nvalid;    // entries in the scored set
  int done;      // finished histogram workgroups
  int nsel;      // entries written to sel
  int ncand;     // entries written to cand
  int pad;
};

struct TopkWs {
  unsigned* hist;    // [T][4096]
  TopkState* st;     // [T]
  int* sel;          // [T][k]
  uint2* cand;       // [T][kCap]  {key, position}
};

static TopkWs carve(void* ws, int T, int k) {
  TopkWs w;
  char* p = (char*)ws;
  w.hist = (unsigned*)p;
  p += align_up((size_t)T * kHistBins * 4, 256);
  w.st = (TopkState*)p;
  p += align_up((size_t)T * sizeof(TopkState), 256);
  w.sel = (int*)p;
  p += align_up((size_t)T * k * 4, 256);
  w.cand = (uint2*)p;
  return w;
}

size_t topk_workspace_bytes(int32_t T, int32_t max_ctx, int32_t k) {
  if (max_ctx <= kSmallN || T == 0) return 0;
  return align_up((size_t)T * kHistBins * 4, 256) + align_up((size_t)T * sizeof(TopkState), 256) +
         align_up((size_t)T * k * 4, 256) + align_up((size_t)T * kCap * 8, 256);
}

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ uint64_t composite(unsigned key, int pos) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (unsigned)pos);
}

__device__ __forceinline__ int ncols_of(const TopkArgs& a, int t, int* b_out) {
  const int b = seq_of_query(a.q_start, a.B, t);
  *b_out = b;
  if (a.cand) return a.n_cand;
  const int len = (int)(a.seq_start[b + 1] - a.seq_start[b]);
  return max(0, min(min(a.q_pos[t], len - 1) + 1, a.max_ctx));
}

__device__ __forceinline__ int pos_of(const TopkArgs& a, int t, int col) {
  return a.cand ? a.cand[(int64_t)t * a.n_cand + col] : col;
}

// Exclusive prefix sum over the block (NT threads); lds needs NT/64 ints.
template <int NT>
__device__ int block_exclusive_scan(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) lds[wave] = x;
  __syncthreads();
  int wbase = 0, tot = 0;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    const int s = lds[i];
    if (i < wave) wbase += s;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return wbase + x - v;
}

// Find the digit d with count(digits > d) < need <= count(digits >= d) in hist[nbins].
// Thread t owns bins nbins-1-t*per .. descending.  Result in sh[0] (digit), sh[1] (above).
template <int NT>
__device__ void block_find_digit(const unsigned* hist, int nbins, int need, int* scan_lds, int* sh) {
  const int per = nbins / NT;
  const int top = nbins - 1 - threadIdx.x * per;
  int local = 0;
  for (int i = 0; i < per; ++i) local += (int)hist[top - i];
  if (threadIdx.x == 0) sh[0] = -1;
  int tot;
  int cum = block_exclusive_scan<NT>(local, scan_lds, &tot);
  for (int i = 0; i < per; ++i) {
    const int h = (int)hist[top - i];
    if (cum < need && need <= cum + h) {
      sh[0] = top - i;
      sh[1] = cum;
    }
    cum += h;
  }
  __syncthreads();
}

// Radix select on composites from `src` (entries whose top `nbits` composite bits
// equal those of `prefix`): returns tau such that exactly `need` of them have c >= tau.
template <int NT, class Src>
__device__ uint64_t radix_refine(const Src& src, int n, int need, uint64_t prefix, int nbits,
                                 unsigned* hist, int* scan_lds, int* sh) {
  while (nbits < 64) {
    const int dbits = min(11, 64 - nbits);
    const int shift = 64 - nbits - dbits;
    const uint64_t dmask = (1ull << dbits) - 1;
    for (int i = threadIdx.x; i < 2048; i += NT) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += NT) {
      uint64_t c;
      if (!src.get(i, &c)) continue;
      if (nbits > 0 && (c >> (64 - nbits)) != (prefix >> (64 - nbits))) continue;
      atomicAdd(&hist[(c >> shift) & dmask], 1u);
    }
    __syncthreads();
    block_find_digit<NT>(hist, 2048, need, scan_lds, sh);
    const int d = sh[0];
    if (d < 0) break;                    // fewer matching entries than `need`: keep what matched
    const int above = sh[1];
    const int inbin = (int)hist[d];
    __syncthreads();
    need -= above;
    prefix |= (uint64_t)d << shift;
    nbits += dbits;
    if (inbin == need) break;
  }
  return prefix;
}

// Wave-aggregated append: returns the slot for lanes with flag set.
__device__ __forceinline__ int wave_append(int* counter, bool flag) {
  const unsigned long long m = __ballot(flag);
  if (m == 0) return -1;
  const int lane = threadIdx.x & 63;
  const int leader = __ffsll((long long)m) - 1;
  int base = 0;
  if (lane == leader) base = atomicAdd(counter, __popcll(m));
  base = __shfl(base, leader);
  return base + __popcll(m & ((1ull << lane) - 1));
}

// Sort n_pad (power of two) ints ascending in LDS.
template <int NT>
__device__ void bitonic_sort(int* arr, int n_pad) {
  for (int size = 2; size <= n_pad; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (n_pad >> 1); i += NT) {
        const int lo = 2 * stride * (i / stride) + (i % stride);
        const int hi = lo + stride;
        const bool asc = (lo & size) == 0;
        const int x = arr[lo], y = arr[hi];
        if ((x > y) == asc) {
          arr[lo] = y;
          arr[hi] = x;
        }
      }
      __syncthreads();
    }
  }
}

__device__ __forceinline__ int pow2_at_least(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}

template <int NT>
__device__ void sort_and_write(int* outl, int cnt, int k, int32_t* dst) {
  const int P = pow2_at_least(max(k, 2));
  for (int i = cnt + threadIdx.x; i < P; i += NT) outl[i] = 0x7FFFFFFF;
  __syncthreads();
  bitonic_sort<NT>(outl, P);
  for (int i = threadIdx.x; i < k; i += NT) dst[i] = i < cnt ? outl[i] : -1;
}

// ------------------------------------------------------------------ short rows

struct LdsKeySrc {
  const unsigned* keys;
  const TopkArgs* a;
  int t;
  __device__ bool get(int i, uint64_t* c) const {
    const unsigned key = keys[i];
    if (key == 0u) return false;
    *c = composite(key, pos_of(*a, t, i));
    return true;
  }
};

__global__ __launch_bounds__(1024) void topk_small_kernel(TopkArgs a) {
  constexpr int NT = 1024;
  __shared__ unsigned keys[kSmallN];
  __shared__ unsigned hist[2048];
  __shared__ int outl[4096];
  __shared__ int scan_lds[NT / 64];
  __shared__ int sh[4];
  const int t = blockIdx.x;
  int b;
  const int ncols = ncols_of(a, t, &b);
  if (threadIdx.x == 0) sh[2] = 0;
  __syncthreads();
  int cnt = 0;
  for (int i = threadIdx.x; i < ncols; i += NT) {
    const unsigned key = score_key(a.scores[(int64_t)t * a.ld + i]);
    keys[i] = key;
    cnt += key != 0u;
  }
  if (cnt) atomicAdd(&sh[2], cnt);
  __syncthreads();
  const int nvalid = sh[2];
  if (threadIdx.x == 0) sh[3] = 0;
  __syncthreads();
  LdsKeySrc src{keys, &a, t};
  uint64_t tau = 0;
  const bool all = nvalid <= a.k;
  if (!all) tau = radix_refine<NT>(src, ncols, a.k, 0ull, 0, hist, scan_lds, sh);
  for (int i0 = 0; i0 < ncols; i0 += NT) {
    const int i = i0 + threadIdx.x;
    uint64_t c = 0;
    const bool v = i < ncols && src.get(i, &c) && (all || c >= tau);
    const int slot = wave_append(&sh[3], v);
    if (v && slot < 4096) outl[slot] = pos_of(a, t, i);
  }
  __syncthreads();
  sort_and_write<NT>(outl, min(sh[3], a.k), a.k, a.idx + (int64_t)t * a.k);
}

// ------------------------------------------------------------------ long rows

__global__ void topk_zero_kernel(unsigned* p, size_t n_words) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n_words;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

__global__ __launch_bounds__(256) void topk_hist_kernel(TopkArgs a, TopkWs w) {
  constexpr int NT = 256;
  __shared__ unsigned hist[kHistBins];
  __shared__ int scan_lds[NT / 64];
  __shared__ int sh[4];
  const int t = blockIdx.y;
  int b;
  const int ncols = ncols_of(a, t, &b);
  const int nch = (ncols + kChunk - 1) / kChunk;
  if ((int)blockIdx.x >= nch) return;
  for (int i = threadIdx.x; i < kHistBins; i += NT) hist[i] = 0;
  if (threadIdx.x == 0) sh[2] = 0;
  __syncthreads();
  const int c0 = blockIdx.x * kChunk, c1 = min(c0 + kChunk, ncols);
  const float* row = a.scores + (int64_t)t * a.ld;
  int cnt = 0;
  for (int i = c0 + threadIdx.x; i < c1; i += NT) {
    const unsigned key = score_key(row[i]);
    if (key) {
      atomicAdd(&hist[key >> 20], 1u);
      ++cnt;
    }
  }
  if (cnt) atomicAdd(&sh[2], cnt);
  __syncthreads();
  unsigned* gh = w.hist + (size_t)t * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += NT)
    if (hist[i]) atomicAdd(&gh[i], hist[i]);
  if (threadIdx.x == 0 && sh[2]) atomicAdd(&w.st[t].nvalid, sh[2]);
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) sh[3] = (atomicAdd(&w.st[t].done, 1) == nch - 1);
  __syncthreads();
  if (!sh[3]) return;
  // last workgroup of this query: find the bin holding the k-th entry
  __threadfence();
  for (int i = threadIdx.x; i < kHistBins; i += NT)
    hist[i] = __hip_atomic_load(&gh[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int nvalid = __hip_atomic_load(&w.st[t].nvalid, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (nvalid <= a.k) {
    if (threadIdx.x == 0) {
      w.st[t].d1 = -1;
      w.st[t].above = nvalid;
      w.st[t].cnt1 = 0;
    }
    return;
  }
  block_find_digit<NT>(hist, kHistBins, a.k, scan_lds, sh);
  if (threadIdx.x == 0) {
    w.st[t].d1 = sh[0];
    w.st[t].above = sh[1];
    w.st[t].cnt1 = (int)hist[sh[0]];
  }
}

__global__ __launch_bounds__(256) void topk_collect_kernel(TopkArgs a, TopkWs w) {
  const int t = blockIdx.y;
  int b;
  const int ncols = ncols_of(a, t, &b);
  const int c0 = blockIdx.x * kChunk;
  if (c0 >= ncols) return;
  const int c1 = min(c0 + kChunk, ncols);
  const int d1 = w.st[t].d1;
  const bool keep_bin = d1 >= 0 && w.st[t].cnt1 <= kCap;
  const float* row = a.scores + (int64_t)t * a.ld;
  int* sel = w.sel + (int64_t)t * a.k;
  uint2* cand = w.cand + (int64_t)t * kCap;
  for (int i0 = c0; i0 < c1; i0 += 256) {
    const int i = i0 + threadIdx.x;
    unsigned key = 0;
    if (i < c1) key = score_key(row[i]);
    const int digit = (int)(key >> 20);
    const bool up = key != 0u && (d1 < 0 || digit > d1);
    const bool in = key != 0u && keep_bin && digit == d1;
    const int s1 = wave_append(&w.st[t].nsel, up);
    if (up) sel[s1] = pos_of(a, t, i);
    const int s2 = wave_append(&w.st[t].ncand, in);
    if (in) cand[s2] = make_uint2(key, (unsigned)pos_of(a, t, i));
  }
}

struct LdsPairSrc {
  const unsigned* keys;
  const int* pos;
  __device__ bool get(int i, uint64_t* c) const {
    *c = composite(keys[i], pos[i]);
    return true;
  }
};

struct GlobalBinSrc {
  const TopkArgs* a;
  int t;
  int d1;
  __device__ bool get(int i, uint64_t* c) const {
    const unsigned key = score_key(a->scores[(int64_t)t * a->ld + i]);
    if (key == 0u || (int)(key >> 20) != d1) return false;
    *c = composite(key, pos_of(*a, t, i));
    return true;
  }
};

__global__ __launch_bounds__(1024) void topk_finish_kernel(TopkArgs a, TopkWs w) {
  constexpr int NT = 1024;
  __shared__ unsigned ck[kCap];
  __shared__ int cp[kCap];
  __shared__ unsigned hist[2048];
  __shared__ int outl[4096];
  __shared__ int scan_lds[NT / 64];
  __shared__ int sh[4];
  const int t = blockIdx.x;
  int b;
  const int ncols = ncols_of(a, t, &b);
  const TopkState st = w.st[t];
  const int above = st.above;
  const int* sel = w.sel + (int64_t)t * a.k;
  for (int i = threadIdx.x; i < above; i += NT) outl[i] = sel[i];
  if (threadIdx.x == 0) sh[3] = above;
  __syncthreads();
  const int need = (st.d1 < 0 || ncols == 0) ? 0 : a.k - above;
  if (need > 0) {
    const uint64_t prefix = (uint64_t)st.d1 << 52;
    if (st.cnt1 <= kCap) {
      const uint2* cand = w.cand + (int64_t)t * kCap;
      const int nc = min(st.ncand, kCap);
      for (int i = threadIdx.x; i < nc; i += NT) {
        const uint2 e = cand[i];
        ck[i] = e.x;
        cp[i] = (int)e.y;
      }
      __syncthreads();
      LdsPairSrc src{ck, cp};
      const uint64_t tau = radix_refine<NT>(src, nc, need, prefix, 12, hist, scan_lds, sh);
      for (int i0 = 0; i0 < nc; i0 += NT) {
        const int i = i0 + threadIdx.x;
        uint64_t c = 0;
        const bool v = i < nc && src.get(i, &c) && c >= tau;
        const int slot = wave_append(&sh[3], v);
        if (v && slot < 4096) outl[slot] = cp[i];
      }
    } else {
      GlobalBinSrc src{&a, t, st.d1};
      const uint64_t tau = radix_refine<NT>(src, ncols, need, prefix, 12, hist, scan_lds, sh);
      for (int i0 = 0; i0 < ncols; i0 += NT) {
        const int i = i0 + threadIdx.x;
        uint64_t c = 0;
        const bool v = i < ncols && src.get(i, &c) && c >= tau;
        const int slot = wave_append(&sh[3], v);
        if (v && slot < 4096) outl[slot] = pos_of(a, t, i);
      }
    }
  }
  __syncthreads();
  sort_and_write<NT>(outl, min(sh[3], a.k), a.k, a.idx + (int64_t)t * a.k);
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.max_ctx <= kSmallN) {
    hipLaunchKernelGGL(topk_small_kernel, dim3(a.T), dim3(1024), 0, s, a);
    return hipGetLastError();
  }
  TopkWs w = carve(a.ws, a.T, a.k);
  const size_t zero_words = ((char*)w.sel - (char*)w.hist) / 4;
  const int zblocks = (int)std::min<size_t>((zero_words + 1023) / 1024, 2048);
  hipLaunchKernelGGL(topk_zero_kernel, dim3(zblocks), dim3(256), 0, s, w.hist, zero_words);
  const int nch = (a.max_ctx + kChunk - 1) / kChunk;
  hipLaunchKernelGGL(topk_hist_kernel, dim3(nch, a.T), dim3(256), 0, s, a, w);
  hipLaunchKernelGGL(topk_collect_kernel, dim3(nch, a.T), dim3(256), 0, s, a, w);
  hipLaunchKernelGGL(topk_finish_kernel, dim3(a.T), dim3(1024), 0, s, a, w);
  return hipGetLastError();
}

}  // namespace smqa
