// Top-k position selection on gfx950 (vLLM blog "DeepSeek-V4.1-Flash sur vLLM",
// sections TL;DR and "Kernels": the DeepSelect top-k over the indexer scores).
//
// Order: score descending, ties to the lower position.  Column i of a query's
// score row stands for position i (dense) or cand[i] (candidate lists are strictly
// ascending), so "lower position" = "lower column".  Every column gets the 64-bit
// composite c = (key(score) << 32) | (0xFFFFFFFF - column), key() being the
// order-preserving float->uint32 map; composites are unique, so the k largest
// composites are exactly the wanted set, found by radix select (11-bit digits,
// most significant first).  The selection is recorded as a bitmap over columns
// and read out in column order, which yields ascending positions without a sort.
//
// Short rows (<= kSmallN columns): one 1024-thread workgroup per query keeps the
// keys in LDS and runs the whole select there.
// Long rows: (1) many workgroups per query build a 4096-bin histogram of the top
// 12 key bits; (2) many workgroups per query each find the bin d1 holding the k-th
// entry from the finished histogram, write the bitmap words of their columns (every
// entry above d1 selected) with wave ballots and append the entries of bin d1 to
// a candidate list; (3) one workgroup per query finishes the select inside d1
// (from LDS, or by re-reading the row when d1 holds more than kCap entries),
// sets those bits, and reads the bitmap out in order.  When the producer of the
// scores already built the histogram (the streaming score kernel), step (1) is
// skipped.
#include "common.h"

namespace smqa {

constexpr int kSmallN = 16384;
constexpr int kChunk = 4096;          // columns per chunk (a long-row workgroup takes 1, 2 or 4)
constexpr int kCap = 12288;           // candidate-list capacity per query (entries of bin d1)
constexpr int kHistBins = kTopkBins;

struct TopkState {
  int d1;        // threshold bin of the top 12 key bits; -1: every valid entry is selected
  int above;     // entries in bins > d1 (all selected)
  int cnt1;      // entries in bin d1
  int nvalid;    // entries in the scored set
  int ncand;     // entries appended to cand
  int ncols;     // columns of the query's row (stored by whoever builds the histogram)
  int pad;
};

struct TopkWs {
  unsigned* hist;    // [T][4096]
  TopkState* st;     // [T]
  uint2* cand;       // [T][kCap]  {key, column}
  unsigned* bits;    // [T][bw]    selection bitmap over columns
  int bw;            // bitmap words per query
};

static int bitmap_words(int max_ctx) { return (max_ctx + kChunk - 1) / kChunk * (kChunk / 32); }

static TopkWs carve(void* ws, int T, int max_ctx) {
  TopkWs w;
  char* p = (char*)ws;
  w.hist = (unsigned*)p;
  p += align_up((size_t)T * kHistBins * 4, 256);
  w.st = (TopkState*)p;
  p += align_up((size_t)T * sizeof(TopkState), 256);
  w.cand = (uint2*)p;
  p += align_up((size_t)T * kCap * 8, 256);
  w.bits = (unsigned*)p;
  w.bw = bitmap_words(max_ctx);
  return w;
}

size_t topk_workspace_bytes(int32_t T, int32_t max_ctx, int32_t k) {
  (void)k;
  if (max_ctx <= kSmallN || T == 0) return 0;
  return align_up((size_t)T * kHistBins * 4, 256) + align_up((size_t)T * sizeof(TopkState), 256) +
         align_up((size_t)T * kCap * 8, 256) + align_up((size_t)T * bitmap_words(max_ctx) * 4, 256);
}

// ------------------------------------------------------------------ helpers

__device__ __forceinline__ uint64_t composite(unsigned key, int col) {
  return ((uint64_t)key << 32) | (uint64_t)(0xFFFFFFFFu - (unsigned)col);
}

__device__ __forceinline__ int ncols_of(const TopkArgs& a, int t) {
  if (a.cand) return a.n_cand;
  const int b = seq_of_query(a.q_start, a.B, t);
  const int len = (int)(a.seq_start[b + 1] - a.seq_start[b]);
  return max(0, min(min(a.q_pos[t], len - 1) + 1, a.max_ctx));
}


// Digit search by one wave: hist[nbins] (nbins = 64 * per), lane l owning the per bins
// below nbins - per * l, in descending order.  Writes sh[0] = d with
// count(bins > d) < need <= count(bins >= d) (-1 if none) and sh[1] = count(bins > d).
template <int PER>
__device__ void wave_find_digit(const unsigned* hist, int need, int* sh) {
  const int lane = threadIdx.x & 63;
  const int top = 64 * PER - 1 - PER * lane;
  unsigned h[PER];
  int local = 0;
#pragma unroll
  for (int i = 0; i < PER; i += 4) {
    const uint4 q = *(const uint4*)(&hist[top - i - 3]);
    h[i] = q.w;
    h[i + 1] = q.z;
    h[i + 2] = q.y;
    h[i + 3] = q.x;
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) local += (int)h[i];
  const int incl = wave_inclusive_sum(local);
  int cum = incl - local;
  const int total = __builtin_amdgcn_readlane(incl, 63);
  if (lane == 0 && total < need) sh[0] = -1;
  if (cum < need && need <= incl) {
#pragma unroll
    for (int i = 0; i < PER; ++i) {
      const int hv = (int)h[i];
      if (cum < need && need <= cum + hv) {
        sh[0] = top - i;
        sh[1] = cum;
      }
      cum += hv;
    }
  }
}

// Exclusive prefix sum over the block (NT threads); lds needs NT/64 ints.
template <int NT>
__device__ int block_exclusive_scan(int v, int* lds, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int x = wave_inclusive_sum(v);
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
// Thread t owns bins nbins-1-t*per .. descending.  Result: sh[0] = digit (-1 if none),
// sh[1] = count above it.
// nbins / NT must be a multiple of 4: each thread reads its bins as 16-byte vectors (lanes
// 16 bytes apart, no bank conflicts when nbins / NT == 4).
template <int NT>
__device__ void block_find_digit(const unsigned* hist, int nbins, int need, int* scan_lds, int* sh) {
  const int per = nbins / NT;
  const int top = nbins - 1 - threadIdx.x * per;
  int local = 0;
  for (int i = 0; i < per; i += 4) {
    const uint4 q = *(const uint4*)&hist[top - i - 3];
    local += (int)(q.x + q.y + q.z + q.w);
  }
  if (threadIdx.x == 0) sh[0] = -1;
  int tot;
  int cum = block_exclusive_scan<NT>(local, scan_lds, &tot);
  for (int i = 0; i < per; i += 4) {
    const uint4 q = *(const uint4*)&hist[top - i - 3];
    const int hv[4] = {(int)q.w, (int)q.z, (int)q.y, (int)q.x};   // bins top-i, top-i-1, ...
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      if (cum < need && need <= cum + hv[u]) {
        sh[0] = top - i - u;
        sh[1] = cum;
      }
      cum += hv[u];
    }
  }
  __syncthreads();
}

// Radix select on composites from `src` restricted to entries whose top `nbits`
// bits equal those of `prefix`: returns tau such that exactly `need` of them have
// c >= tau.  Digits of DBITS bits (hist holds 2^DBITS bins).  SKIP_COMMON first finds
// the leading bits shared by every matching entry (one extra pass over the source) and
// starts the digits below them: worth it when a pass is expensive (a global row).
template <int NT, int DBITS, bool SKIP_COMMON, class Src>
__device__ uint64_t radix_refine(const Src& src, int n, int need, uint64_t prefix, int nbits,
                                 unsigned* hist, int* scan_lds, int* sh) {
  constexpr int NBINS = 1 << DBITS;
  static_assert(NBINS % (4 * NT) == 0, "block_find_digit reads 4 bins per vector");
  if (SKIP_COMMON) {
    uint64_t lo = ~0ull, hi = 0ull;
    for (int i = threadIdx.x; i < n; i += NT) {
      uint64_t c;
      if (!src.get(i, &c)) continue;
      if (nbits > 0 && (c >> (64 - nbits)) != (prefix >> (64 - nbits))) continue;
      lo = c < lo ? c : lo;
      hi = c > hi ? c : hi;
    }
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const uint64_t l2 = __shfl_xor(lo, o), h2 = __shfl_xor(hi, o);
      lo = l2 < lo ? l2 : lo;
      hi = h2 > hi ? h2 : hi;
    }
    uint64_t* red = (uint64_t*)hist;      // hist is free here
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    if (lane == 0) {
      red[2 * wave] = lo;
      red[2 * wave + 1] = hi;
    }
    __syncthreads();
    lo = ~0ull;
    hi = 0ull;
    for (int i = 0; i < NT / 64; ++i) {
      lo = red[2 * i] < lo ? red[2 * i] : lo;
      hi = red[2 * i + 1] > hi ? red[2 * i + 1] : hi;
    }
    __syncthreads();
    if (lo <= hi) {
      const int common = lo == hi ? 64 : __clzll((long long)(lo ^ hi));
      if (common > nbits) {
        prefix = common == 64 ? lo : (lo >> (64 - common)) << (64 - common);
        nbits = common;
      }
    }
  }
  while (nbits < 64) {
    const int dbits = min(DBITS, 64 - nbits);
    const int shift = 64 - nbits - dbits;
    const uint64_t dmask = (1ull << dbits) - 1;
    for (int i = threadIdx.x; i < NBINS; i += NT) hist[i] = 0;
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += NT) {
      uint64_t c;
      if (!src.get(i, &c)) continue;
      if (nbits > 0 && (c >> (64 - nbits)) != (prefix >> (64 - nbits))) continue;
      atomicAdd(&hist[(c >> shift) & dmask], 1u);
    }
    __syncthreads();
    block_find_digit<NT>(hist, NBINS, need, scan_lds, sh);
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

// Wave-aggregated append to an LDS or global counter: returns this lane's slot.
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

// Read the selection out in column order: dst[i] = position of the i-th selected column,
// then -1 up to k.  Selected = the bits of `bits` (nwords words over the columns, written by
// an earlier kernel) plus the nwin columns win[] (in LDS).  Rounds of NT*PER words: each
// thread puts its PER consecutive words in the LDS bitmap `lbits` (transposed: word j of
// thread i at j * NT + i, so every access of a wave is conflict-free), the round's winners
// are OR-ed in, and one block scan of the per-thread bit counts gives each thread the output
// offset of its first bit.  Each nonzero word whose first bit is an output is then filed
// under that offset as one 8-byte pair in `fw` (its bits and its first column; kMaxK
// entries, the bits cleared to 0 beforehand), and the output slots are shared out over the
// threads: the thread of a
// slot where a word starts writes that word's columns to the LDS staging array `out`.  A
// thread's loop then runs over the bits of one word, not over every bit of its PER words
// (a short row leaves most threads without words and a few with hundreds of bits).  The
// round's outputs are copied to dst with coalesced stores (positions looked up in the
// candidate list there, in parallel).  first[] holds this thread's words of the first round,
// loaded by the caller in advance (garbage past nwords is masked here).
constexpr int kSelPer = 16;
constexpr int kMaxK = 4096;            // the largest k the read-out stages
template <int NT>
__device__ void write_selection(const TopkArgs& a, int t, const unsigned* bits, int nwords,
                                const uint4 (&first)[kSelPer / 4], const int* win, int nwin,
                                unsigned* lbits, uint2* fw, int* out, int32_t* dst, int* scan_lds) {
  constexpr int PER = kSelPer;
  int done = 0;
  for (int r0 = 0; r0 < nwords && done < a.k; r0 += NT * PER) {
    const int w0 = r0 + threadIdx.x * PER;
    // w0 is a multiple of 16 and the per-query bitmap a multiple of 128 words, so a group
    // that starts below nwords lies inside it
    uint4 g4[PER / 4];
#pragma unroll
    for (int j = 0; j < PER / 4; ++j)
      g4[j] = r0 == 0 ? first[j] : w0 < nwords ? *(const uint4*)(bits + w0 + 4 * j) : make_uint4(0u, 0u, 0u, 0u);
    unsigned wv[PER];
#pragma unroll
    for (int j = 0; j < PER / 4; ++j) {
      wv[4 * j] = g4[j].x;
      wv[4 * j + 1] = g4[j].y;
      wv[4 * j + 2] = g4[j].z;
      wv[4 * j + 3] = g4[j].w;
    }
#pragma unroll
    for (int j = 0; j < PER; ++j)
      if (w0 + j >= nwords) wv[j] = 0u;
    if (nwin > 0) {                      // uniform
#pragma unroll
      for (int j = 0; j < PER; ++j) lbits[j * NT + threadIdx.x] = wv[j];
      __syncthreads();
      for (int i = threadIdx.x; i < nwin; i += NT) {
        const int wi = (win[i] >> 5) - r0;
        if (wi >= 0 && wi < NT * PER) atomicOr(&lbits[(wi % PER) * NT + wi / PER], 1u << (win[i] & 31));
      }
      __syncthreads();
#pragma unroll
      for (int j = 0; j < PER; ++j) wv[j] = lbits[j * NT + threadIdx.x];
    }
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) cnt += __popc(wv[j]);
    for (int i = threadIdx.x; i < kMaxK; i += NT) fw[i].x = 0u;
    // (the block scan's barriers order the clearing before the filing below)
    int total;
    int off = block_exclusive_scan<NT>(cnt, scan_lds, &total);
    const int nout = min(total, a.k - done);
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      if (wv[j] != 0u && off < nout) fw[off] = make_uint2(wv[j], (unsigned)(32 * (w0 + j)));
      off += __popc(wv[j]);
    }
    __syncthreads();
    for (int o = threadIdx.x; o < nout; o += NT) {
      const uint2 f = fw[o];
      unsigned m = f.x;
      const int c0 = (int)f.y;
      int p = o;
      while (m && p < nout) {
        out[p++] = c0 + __ffs(m) - 1;
        m &= m - 1;
      }
    }
    __syncthreads();
    float* vdst = a.val ? a.val + (int64_t)t * a.k : nullptr;
    for (int o = threadIdx.x; o < nout; o += NT) {
      const int col = out[o];
      dst[done + o] = a.cand ? a.cand[(int64_t)t * a.n_cand + col] : col;
      if (vdst) vdst[done + o] = a.scores[(int64_t)t * a.ld + col];
    }
    done += nout;
    __syncthreads();                     // lbits and out are rewritten by the next round
  }
  for (int i = done + threadIdx.x; i < a.k; i += NT) {
    dst[i] = -1;
    if (a.val) a.val[(int64_t)t * a.k + i] = -__builtin_inff();
  }
}

// ------------------------------------------------------------------ short rows

// One 1024-thread workgroup per query.  Thread i owns columns PER i .. PER i + PER - 1
// (keys staged through LDS so the row is read with coalesced loads) and keeps their 32-bit
// keys in registers; PER = 8 for rows of at most 8192 columns, else 16 (the work per
// column is VALU-bound on one CU, so a row is not padded to the larger width).  Radix select over the keys finds tau with count(key > tau) < k <=
// count(key >= tau); when several columns share the key tau, the lowest columns among
// them are taken.  Column order is thread order, so one block-wide scan of a packed
// (ties, greater) count pair yields both each thread's tie rank and its output offset,
// and the selection comes out in ascending column order.
template <int PER>
__global__ __launch_bounds__(1024) void topk_small_kernel(TopkArgs a) {
  constexpr int NT = 1024;
  constexpr int N = NT * PER;                     // columns of the row this instance handles
  static_assert(PER % 4 == 0 && N <= kSmallN, "keys are read back as 16-byte vectors");
  __shared__ __attribute__((aligned(16))) unsigned keys[N];
  __shared__ __attribute__((aligned(16))) unsigned hist[2048];
  __shared__ unsigned red[2 * (NT / 64)];
  __shared__ int scan_lds[NT / 64];
  __shared__ int sh[4];
  const int t = blockIdx.x, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const float* row = a.scores + (int64_t)t * a.ld;
  static_assert(2 * NT == 2048, "two histogram bins per thread");
  // row loads first (bounded by the row width, known without any load), the query's
  // column count (a chain of small dependent loads) meanwhile
  float v[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int col = tid + NT * u;
    v[u] = col < a.max_ctx ? row[col] : -__builtin_inff();
  }
  const int ncols = ncols_of(a, t);
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    const int col = tid + NT * u;
    keys[col] = col < ncols ? score_key(v[u]) : 0u;
  }
  hist[2 * tid] = 0u;                              // zero for the first radix pass
  hist[2 * tid + 1] = 0u;
  __syncthreads();
  unsigned key[PER];
#pragma unroll
  for (int u = 0; u < PER; u += 4) {
    const uint4 k4 = *(const uint4*)(&keys[PER * tid + u]);
    key[u] = k4.x;
    key[u + 1] = k4.y;
    key[u + 2] = k4.z;
    key[u + 3] = k4.w;
  }
  const int c0 = PER * tid;
  // valid count and the min / max valid key (min as the max of ~key over valid keys)
  int cnt = 0;
  unsigned nlo = 0u, hi = 0u;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    cnt += key[u] != 0u;
    nlo = key[u] ? max(nlo, ~key[u]) : nlo;
    hi = max(hi, key[u]);
  }
  cnt = wave_inclusive_sum(cnt);
  nlo = wave_inclusive_max(nlo);
  hi = wave_inclusive_max(hi);
  if (lane == 63) {
    scan_lds[wave] = cnt;
    red[2 * wave] = nlo;
    red[2 * wave + 1] = hi;
  }
  __syncthreads();
  int nvalid = 0;
  nlo = 0u;
  hi = 0u;
#pragma unroll
  for (int i = 0; i < NT / 64; ++i) {
    nvalid += scan_lds[i];
    nlo = max(nlo, red[2 * i]);
    hi = max(hi, red[2 * i + 1]);
  }
  unsigned lo = ~nlo;
  __syncthreads();

  unsigned tau = 1u;                               // every valid key is >= 1
  int tie_need = NT * PER;                         // columns with key == tau to take
  if (nvalid > a.k) {
    // leading bits shared by every valid key carry no information
    int nbits = lo == hi ? 32 : __clz((int)(lo ^ hi));
    unsigned prefix = nbits == 32 ? lo : (nbits == 0 ? 0u : (lo >> (32 - nbits)) << (32 - nbits));
    int need = a.k;
    bool whole_bin = false;
    while (nbits < 32) {
      const int dbits = min(11, 32 - nbits);
      const int shift = 32 - nbits - dbits;
      const unsigned dmask = (1u << dbits) - 1u;
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const bool match = key[u] != 0u && (nbits == 0 || (key[u] >> (32 - nbits)) == (prefix >> (32 - nbits)));
        if (match) atomicAdd(&hist[(key[u] >> shift) & dmask], 1u);
      }
      __syncthreads();
      // the digit, over the whole block: thread i holds bins 2047 - 2i and 2046 - 2i (the
      // bins count down with the thread index, so a prefix sum counts the keys above)
      const int h1 = (int)hist[2047 - 2 * tid], h0 = (int)hist[2046 - 2 * tid];
      const int local = h1 + h0;
      const int incl = wave_inclusive_sum(local);
      if (lane == 63) scan_lds[wave] = incl;
      if (tid == 0) sh[0] = -1;
      __syncthreads();
      int cum = incl - local;
#pragma unroll
      for (int i = 0; i < NT / 64; ++i)
        if (i < wave) cum += scan_lds[i];
      if (cum < need && need <= cum + local) {
        const bool upper = need <= cum + h1;
        sh[0] = upper ? 2047 - 2 * tid : 2046 - 2 * tid;
        sh[1] = upper ? cum : cum + h1;
        sh[2] = upper ? h1 : h0;
      }
      hist[2 * tid] = 0u;                          // every bin was read before the barrier
      hist[2 * tid + 1] = 0u;
      __syncthreads();
      const int d = sh[0];
      if (d < 0) break;                            // cannot happen: nvalid > k
      const int above = sh[1];
      const int inbin = sh[2];
      need -= above;
      prefix |= (unsigned)d << shift;
      nbits += dbits;
      if (inbin == need) {                         // the whole bin is taken
        whole_bin = true;
        break;
      }
    }
    tau = max(prefix, 1u);                         // a bin's lower bound may be the invalid key 0
    if (!whole_bin) tie_need = need;               // tau fully resolved: `need` of its ties
  }
  // (ties, greater) counts packed in one scan: both fit in 16 bits
  int ngt = 0, nties = 0;
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    ngt += key[u] > tau;
    nties += key[u] == tau;
  }
  int total;
  const int pre = block_exclusive_scan<NT>((nties << 16) | ngt, scan_lds, &total);
  int tie_rank = pre >> 16;
  int off = (pre & 0xFFFF) + min(tie_rank, tie_need);
  const int nsel = (total & 0xFFFF) + min(total >> 16, tie_need);
  int32_t* dst = a.idx + (int64_t)t * a.k;
  // positions first (a candidate list is read before any store), then the stores
  int pos[PER];
#pragma unroll
  for (int u = 0; u < PER; ++u) pos[u] = c0 + u;
  if (a.cand) {
#pragma unroll
    for (int u = 0; u < PER; ++u)
      if (c0 + u < a.n_cand) pos[u] = a.cand[(int64_t)t * a.n_cand + c0 + u];
  }
  // the selection is staged in LDS (the key array is free: the keys are in registers)
  // and written out with coalesced stores
  // (scores, when asked for, are the exact inverses of the keys, staged next to them)
  int* stage = (int*)keys;
  float* vstage = (float*)(keys + 4096);
  static_assert(N >= 2 * 4096, "position and score staging for k <= 4096");
#pragma unroll
  for (int u = 0; u < PER; ++u) {
    bool sel = key[u] > tau;
    if (key[u] == tau) sel = tie_rank++ < tie_need;
    if (sel) {
      if (off < a.k) {
        stage[off] = pos[u];
        if (a.val) vstage[off] = key_score(key[u]);
      }
      ++off;
    }
  }
  __syncthreads();
  for (int i = tid; i < a.k; i += NT) dst[i] = i < nsel ? stage[i] : -1;
  if (a.val) {
    float* vdst = a.val + (int64_t)t * a.k;
    for (int i = tid; i < a.k; i += NT) vdst[i] = i < nsel ? vstage[i] : -__builtin_inff();
  }
}

// ------------------------------------------------------------------ long rows

__global__ void topk_zero_kernel(unsigned* p, size_t n_words) {
  for (size_t i = blockIdx.x * (size_t)blockDim.x + threadIdx.x; i < n_words;
       i += (size_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

constexpr int kLongThreads = 256;
constexpr int kPerThread = kChunk / kLongThreads;

struct Threshold {
  int d1, above, cnt1;
};

// A workgroup counts HC consecutive chunks of a row into one LDS histogram before adding its
// nonzero bins to the query's global one: on long rows the global atomics, not the row
// reads, bound this kernel (HC = 4 from 20 chunks per row on; shorter rows keep one chunk
// per workgroup for parallelism).
template <int HC>
__global__ __launch_bounds__(kLongThreads) void topk_hist_kernel(TopkArgs a, TopkWs w) {
  constexpr int NT = kLongThreads;
  __shared__ unsigned hist[kHistBins];
  const int t = blockIdx.y;
  const int c0 = blockIdx.x * HC * kChunk;
  const float* row = a.scores + (int64_t)t * a.ld;
  // every load of the workgroup's columns goes out first, bounded by the row width (known
  // without any load; the grid covers it), while the query's column count (a chain of small
  // dependent loads) is read; columns past that count are masked afterwards
  float v[HC * kPerThread];
#pragma unroll
  for (int u = 0; u < HC * kPerThread; ++u) {
    const int i = c0 + threadIdx.x + NT * u;
    v[u] = i < a.max_ctx ? row[i] : -__builtin_inff();
  }
  const int ncols = ncols_of(a, t);
  if (blockIdx.x == 0 && threadIdx.x == 0) w.st[t].ncols = ncols;
  const int nch = (ncols + HC * kChunk - 1) / (HC * kChunk);
  if ((int)blockIdx.x >= nch) return;
  for (int i = threadIdx.x; i < kHistBins; i += NT) hist[i] = 0;
  __syncthreads();
#pragma unroll
  for (int u = 0; u < HC * kPerThread; ++u) {
    const unsigned key = c0 + (int)threadIdx.x + NT * u < ncols ? score_key(v[u]) : 0u;
    if (key) atomicAdd(&hist[key >> 20], 1u);
  }
  __syncthreads();
  // the nonzero bins into the query's global histogram; the collect kernel, launched after
  // this one completes, finds the threshold bin from it
  unsigned* gh = w.hist + (size_t)t * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += NT)
    if (hist[i]) atomicAdd(&gh[i], hist[i]);
}

// The query's histogram was completed by an earlier kernel (the histogram kernel, or the
// streaming score kernel); each workgroup reads it (16 KB, issued with the row loads) and
// finds d1 itself, and the query's first chunk publishes it for the finish kernel.  A
// workgroup takes HC consecutive chunks (HC = 2 when a call has thousands of chunks, so the
// histogram read and the threshold scan are paid once per two chunks; one chunk otherwise,
// for parallelism).  Its candidates (entries of bin d1) go to the query's list with one
// atomic per workgroup: staged in LDS with one chunk, written straight from registers after
// a block scan of the per-thread counts with two (an LDS stage for two chunks would cost
// occupancy).
template <int HC>
__global__ __launch_bounds__(kLongThreads) void topk_collect_kernel(TopkArgs a, TopkWs w) {
  constexpr int NT = kLongThreads;
  constexpr int NV = HC * kPerThread;
  __shared__ uint2 buf[HC == 1 ? kChunk : 1];
  __shared__ int scan_lds[NT / 64];
  __shared__ int sh[4];
  __shared__ int nbuf, gbase;
  const int t = blockIdx.y;
  const int c0 = blockIdx.x * HC * kChunk;
  const float* row = a.scores + (int64_t)t * a.ld;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // Every load is issued before the query's column count arrives: the row bounded by the
  // host's max_ctx (<= ld), then masked to the query's own count.
  // wave `wave`, step u covers columns c0 + 64*(wave + 4u) + lane
  const TopkState st0 = w.st[t];
  float v[NV];
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int i = c0 + 64 * (wave + 4 * u) + lane;
    v[u] = i < a.max_ctx ? row[i] : -__builtin_inff();
  }
  int d1, cnt1;
  {
    // Thread i holds bins [16i, 16i + 16) in registers (four 16-byte loads; the histogram
    // was completed by an earlier kernel, so plain loads see it).  One block scan of the
    // per-thread counts gives the total and, as total - prefix - own, the count above each
    // thread's bins, so the thread holding the k-th entry finds d1 in its own registers.
    constexpr int PER = kHistBins / NT;
    const uint4* gh = (const uint4*)(w.hist + (size_t)t * kHistBins + PER * threadIdx.x);
    uint4 h4[PER / 4];
#pragma unroll
    for (int j = 0; j < PER / 4; ++j) h4[j] = gh[j];
    if (threadIdx.x == 0) h4[0].x = 0u;                 // bin 0 holds only key 0 (not scored)
    unsigned hv[PER];
#pragma unroll
    for (int j = 0; j < PER / 4; ++j) {
      hv[4 * j] = h4[j].x;
      hv[4 * j + 1] = h4[j].y;
      hv[4 * j + 2] = h4[j].z;
      hv[4 * j + 3] = h4[j].w;
    }
    int cnt = 0;
#pragma unroll
    for (int j = 0; j < PER; ++j) cnt += (int)hv[j];
    if (c0 >= st0.ncols) return;                     // uniform: before any barrier
    if (threadIdx.x == 0) sh[0] = -1;
    int nvalid;
    const int pre = block_exclusive_scan<NT>(cnt, scan_lds, &nvalid);
    if (nvalid > a.k) {
      int above = nvalid - pre - cnt;
      if (above < a.k && a.k <= above + cnt) {
#pragma unroll
        for (int j = PER - 1; j >= 0; --j) {
          if (above < a.k && a.k <= above + (int)hv[j]) {
            sh[0] = PER * threadIdx.x + j;
            sh[1] = above;
            sh[2] = (int)hv[j];
          }
          above += (int)hv[j];
        }
      }
    }
    __syncthreads();
    const Threshold th = nvalid <= a.k ? Threshold{-1, nvalid, 0} : Threshold{sh[0], sh[1], sh[2]};
    d1 = th.d1;
    cnt1 = th.cnt1;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
      w.st[t].d1 = th.d1;
      w.st[t].above = th.above;
      w.st[t].cnt1 = th.cnt1;
      w.st[t].nvalid = nvalid;
    }
  }
  const int ncols = st0.ncols;
#pragma unroll
  for (int u = 0; u < NV; ++u)
    if (c0 + 64 * (wave + 4 * u) + lane >= ncols) v[u] = -__builtin_inff();
  const bool keep_bin = d1 >= 0 && cnt1 <= kCap;
  unsigned* bits = w.bits + (size_t)t * w.bw;
  const int bcols = 32 * w.bw;                       // columns the query's bitmap covers
  int cin = 0;
  if (HC == 1) {
    if (threadIdx.x == 0) nbuf = 0;
    __syncthreads();
  }
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    const int cb = c0 + 64 * (wave + 4 * u);
    const unsigned key = score_key(v[u]);
    const int digit = (int)(key >> 20);
    const bool up = key != 0u && (d1 < 0 || digit > d1);
    const bool in = key != 0u && keep_bin && digit == d1;
    const unsigned long long m = __ballot(up);
    if (lane == 0 && cb < bcols) {                   // (a last workgroup's chunks may pass it)
      bits[cb / 32] = (unsigned)m;
      bits[cb / 32 + 1] = (unsigned)(m >> 32);
    }
    if constexpr (HC == 1) {
      const int slot = wave_append(&nbuf, in);
      if (in) buf[slot] = make_uint2(key, (unsigned)(cb + lane));
    } else {
      cin += in;
    }
  }
  if constexpr (HC == 1) {
    // one chunk: the candidates were staged in LDS, one atomic and a coalesced copy
    __syncthreads();
    const int nb = nbuf;
    if (nb == 0) return;
    if (threadIdx.x == 0) gbase = atomicAdd(&w.st[t].ncand, nb);
    __syncthreads();
    uint2* cand = w.cand + (int64_t)t * kCap;
    for (int i = threadIdx.x; i < nb; i += NT)
      if (gbase + i < kCap) cand[gbase + i] = buf[i];
    return;
  }
  int ntot;
  int off = block_exclusive_scan<NT>(cin, scan_lds, &ntot);
  if (ntot == 0) return;                             // uniform
  if (threadIdx.x == 0) gbase = atomicAdd(&w.st[t].ncand, ntot);
  __syncthreads();
  off += gbase;
  uint2* cand = w.cand + (int64_t)t * kCap;
#pragma unroll
  for (int u = 0; u < NV; ++u) {
    // (the key is recomputed rather than kept from the first pass: 64 more live registers
    // would cut the workgroups per CU)
    float x = v[u];
    asm volatile("" : "+v"(x));
    const unsigned key = score_key(x);
    if (key != 0u && keep_bin && (int)(key >> 20) == d1) {
      if (off < kCap) cand[off] = make_uint2(key, (unsigned)(c0 + 64 * (wave + 4 * u) + lane));
      ++off;
    }
  }
}

// Chunks per collect workgroup: two once a call has thousands of chunks (the replay chunk's
// 25,600: 348 -> 308 us for the top-k; four chunks held 199 registers and were slower), else
// one.
static hipError_t launch_collect(const TopkArgs& a, const TopkWs& w, int nch, hipStream_t s) {
  if ((int64_t)nch * a.T >= 4096)
    hipLaunchKernelGGL(topk_collect_kernel<2>, dim3((nch + 1) / 2, a.T), dim3(kLongThreads), 0, s, a, w);
  else
    hipLaunchKernelGGL(topk_collect_kernel<1>, dim3(nch, a.T), dim3(kLongThreads), 0, s, a, w);
  return hipGetLastError();
}

struct LdsPairSrc {
  const unsigned* keys;
  const int* cols;
  __device__ bool get(int i, uint64_t* c) const {
    *c = composite(keys[i], cols[i]);
    return true;
  }
};

struct GlobalBinSrc {
  const float* row;
  int d1;
  __device__ bool get(int i, uint64_t* c) const {
    const unsigned key = score_key(row[i]);
    if (key == 0u || (int)(key >> 20) != d1) return false;
    *c = composite(key, i);
    return true;
  }
};

// One workgroup per query: the select inside the threshold bin d1 (need = k - above of its
// entries), then the read-out.  The bin's entries come from the candidate list (in LDS)
// or, when it overflowed, from the row itself.  Winners are collected in LDS, and the
// read-out merges them with the collect kernel's bitmap, so nothing is written to global
// memory and read back.
constexpr int kRefineBits = 12;
__global__ __launch_bounds__(1024) void topk_finish_kernel(TopkArgs a, TopkWs w) {
  constexpr int NT = 1024;
  // ck | cc while refining, then the read-out's LDS bitmap (2 * kCap >= NT * 16 words)
  __shared__ __attribute__((aligned(16))) unsigned pool[2 * kCap];
  // refine histogram, then the winners' columns (need <= k <= 4096 of them)
  __shared__ __attribute__((aligned(16))) unsigned hist[1 << kRefineBits];
  __shared__ int scan_lds[NT / 64];
  __shared__ int sh[4];
  __shared__ int nwin;
  __shared__ int out[kMaxK];          // read-out staging (k <= 4096)
  // the read-out's LDS bitmap (NT * kSelPer words), then its filed words and columns
  static_assert(2 * kCap >= NT * kSelPer + 2 * kMaxK, "read-out bitmap does not fit");
  unsigned* ck = pool;
  int* cc = (int*)(pool + kCap);
  int* win = (int*)hist;
  const int t = blockIdx.x;
  const unsigned* bits = w.bits + (size_t)t * w.bw;
  const float* row = a.scores + (int64_t)t * a.ld;
  const uint2* cand = w.cand + (int64_t)t * kCap;
  // Loads that need nothing from the state go out with it: the read-out's first-round
  // bitmap words (inside the query's bw words whenever the group starts inside them) and
  // the first kPre candidates of the list (inside its kCap slots).
  constexpr int kPre = 3;
  const TopkState st = w.st[t];
  // (a thread past the bitmap loads its last words instead, so every load is issued
  // without a branch; the read-out masks words past the row's count)
  uint4 first[kSelPer / 4];
  {
    const int fw = min(kSelPer * (int)threadIdx.x, w.bw - kSelPer);
#pragma unroll
    for (int j = 0; j < kSelPer / 4; ++j) first[j] = *(const uint4*)(bits + fw + 4 * j);
  }
  uint2 pre[kPre];
#pragma unroll
  for (int j = 0; j < kPre; ++j) pre[j] = cand[threadIdx.x + NT * j];
  const int ncols = st.ncols;
  const int need = (st.d1 < 0 || ncols == 0) ? 0 : a.k - st.above;
  if (threadIdx.x == 0) nwin = 0;
  if (need > 0) {
    const uint64_t prefix = (uint64_t)st.d1 << 52;
    if (st.cnt1 <= kCap) {
      const int nc = min(st.ncand, kCap);
#pragma unroll
      for (int j = 0; j < kPre; ++j) {
        const int i = threadIdx.x + NT * j;
        if (i < nc) {
          ck[i] = pre[j].x;
          cc[i] = (int)pre[j].y;
        }
      }
      for (int i = threadIdx.x + NT * kPre; i < nc; i += NT) {
        const uint2 e = cand[i];
        ck[i] = e.x;
        cc[i] = (int)e.y;
      }
      __syncthreads();
      LdsPairSrc src{ck, cc};
      const uint64_t tau = radix_refine<NT, kRefineBits, false>(src, nc, need, prefix, 12, hist, scan_lds, sh);
      for (int i0 = 0; i0 < nc; i0 += NT) {
        const int i = i0 + threadIdx.x;
        uint64_t c = 0;
        if (i < nc) src.get(i, &c);
        const int slot = wave_append(&nwin, i < nc && c >= tau);
        if (slot >= 0 && i < nc && c >= tau) win[slot] = cc[i];
      }
    } else {
      GlobalBinSrc src{row, st.d1};
      const uint64_t tau = radix_refine<NT, kRefineBits, true>(src, ncols, need, prefix, 12, hist, scan_lds, sh);
      for (int i0 = 0; i0 < ncols; i0 += NT) {
        const int i = i0 + threadIdx.x;
        uint64_t c = 0;
        const bool sel = i < ncols && src.get(i, &c) && c >= tau;
        const int slot = wave_append(&nwin, sel);
        if (sel) win[slot] = i;
      }
    }
  }
  __syncthreads();
  write_selection<NT>(a, t, bits, (ncols + 31) / 32, first, win, nwin, pool, (uint2*)(pool + NT * kSelPer),
                      out, a.idx + (int64_t)t * a.k, scan_lds);
}

hipError_t launch_topk(const TopkArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.max_ctx <= kSmallN) {
    if (a.max_ctx <= 8192) hipLaunchKernelGGL(topk_small_kernel<8>, dim3(a.T), dim3(1024), 0, s, a);
    else hipLaunchKernelGGL(topk_small_kernel<16>, dim3(a.T), dim3(1024), 0, s, a);
    return hipGetLastError();
  }
  TopkFill fill;
  hipError_t e = launch_topk_prepare(a, s, &fill);
  if (e != hipSuccess) return e;
  TopkWs w = carve(a.ws, a.T, a.max_ctx);
  const int nch = (a.max_ctx + kChunk - 1) / kChunk;
  if (nch >= 20) {
    hipLaunchKernelGGL(topk_hist_kernel<4>, dim3((nch + 3) / 4, a.T), dim3(kLongThreads), 0, s, a, w);
  } else {
    hipLaunchKernelGGL(topk_hist_kernel<1>, dim3(nch, a.T), dim3(kLongThreads), 0, s, a, w);
  }
  launch_collect(a, w, nch, s);
  hipLaunchKernelGGL(topk_finish_kernel, dim3(a.T), dim3(1024), 0, s, a, w);
  return hipGetLastError();
}

hipError_t launch_topk_prepare(const TopkArgs& a, hipStream_t s, TopkFill* fill) {
  *fill = TopkFill{nullptr, nullptr, 0};
  if (a.T == 0 || a.max_ctx <= kSmallN) return hipSuccess;
  TopkWs w = carve(a.ws, a.T, a.max_ctx);
  // histogram and per-query state (counters start at zero)
  const size_t zero_words = ((char*)w.cand - (char*)w.hist) / 4;
  const int zblocks = (int)std::min<size_t>((zero_words + 1023) / 1024, 2048);
  hipLaunchKernelGGL(topk_zero_kernel, dim3(zblocks), dim3(256), 0, s, w.hist, zero_words);
  static_assert(sizeof(TopkState) % 4 == 0, "state stride in ints");
  *fill = TopkFill{w.hist, &w.st[0].ncols, (int32_t)(sizeof(TopkState) / 4)};
  return hipGetLastError();
}

hipError_t launch_topk_from_hist(const TopkArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.max_ctx <= kSmallN) return launch_topk(a, s);
  TopkWs w = carve(a.ws, a.T, a.max_ctx);
  const int nch = (a.max_ctx + kChunk - 1) / kChunk;
  launch_collect(a, w, nch, s);
  hipLaunchKernelGGL(topk_finish_kernel, dim3(a.T), dim3(1024), 0, s, a, w);
  return hipGetLastError();
}

}  // namespace smqa
