// Split-K paged attention for q = 1 decode and the short verify window.
//
// Two launches serve both entry points (KAP paper: proposal steps are
// decode-like forwards over the compact view; the verifier scores a short
// window over the full KV with the original positions):
//   1. partial: one wave per work item = (request, KV head, chunk of pages,
//               slice of up to 64 query rows).  Each wave derives its own item
//               from the per-row lengths on the device (closed-form plan, no
//               host synchronization, so calls are graph-capturable) and
//               rotates its own query rows at their logical positions (fp64
//               angles).  All query rows that share a KV head (the GQA group
//               times the window) are processed together, so every K/V byte
//               is read once per item.
//   2. merge  : log-sum-exp combine of a (request, KV head)'s partials in item
//               order (deterministic).
//
// bf16 path: QK^T and PV run on MFMA.  S^T = K Q^T with
// v_mfma_f32_16x16x32_bf16 (A = 16 tokens x 32 dims of K straight from the
// page, B = 32 dims x 16 query rows), which leaves each lane holding one query
// row and 4 tokens of the page.  Pages go in pairs: the lane's 4 + 4
// probabilities of the two pages form the B operand of P^T for O^T = V^T P^T
// on the same 16x16x32 instruction (contraction over the pair's 32 tokens).
// V pages are stored dim-major, so the V^T operand (one dim, 4 consecutive
// tokens of each page) is two contiguous 8-byte loads and no transpose is
// needed anywhere.  The output accumulator holds one query row per lane, so
// the online-softmax rescale is local.
// fp32 path: plain VALU loops (used for the small fp32 workloads).
#include "kap_internal.h"

namespace kap {

// ------------------------------------------------------------------ workspace
AttnWorkspace carve_attn_workspace(void* base, int32_t B, int32_t q_len, int32_t Hq,
                                   int32_t Hkv, int32_t D) {
  AttnWorkspace w{};
  const int32_t grp = Hq / Hkv;
  const int64_t R = (int64_t)grp * q_len;
  w.max_items = kTargetItems + B * Hkv;
  size_t off = 0;
  char* p = (char*)base;
  auto take = [&](size_t bytes) {
    char* r = p ? p + off : nullptr;
    off = align_up(off + bytes, 256);
    return r;
  };
  w.n_items = (int32_t*)take(sizeof(int32_t));
  w.row_off = (int32_t*)take(sizeof(int32_t) * ((size_t)B * Hkv + 1));
  w.part_ml = (float2*)take(sizeof(float2) * (size_t)w.max_items * R);
  w.part_o = (float*)take(sizeof(float) * (size_t)w.max_items * R * D);
  w.bytes = off;
  return w;
}

// ------------------------------------------------------------------ work plan
// Rows are (request b, KV head g); row r reads table row (b, g or 0).  A row
// of np pages is cut into ceil(np / chunk) items of chunk pages, with chunk
// chosen so that the items number at most target (see plan_find); items are
// numbered row by row.  target is the number of waves the partial kernel keeps resident on the
// device (CUs x resident blocks per CU), so a call runs as one round of equal
// items.  Every wave evaluates this closed form for its own item id, so no
// separate planning launch is needed.  At most target + rows items.
struct PlanIn {
  const int32_t* lens;
  int32_t B, Hkv, G, width;
  int32_t target;  // items aimed at: the kernel's resident-wave capacity (<= kTargetItems)
};

// Length entry of row r as stored, and clamped to the table width.
__device__ __forceinline__ int plan_row_raw(const PlanIn& p, int r) {
  const int b = r / p.Hkv, g = r % p.Hkv;
  const int gr = p.G == 1 ? 0 : g;
  return p.lens[b * p.G + gr];
}
__device__ __forceinline__ int plan_clamp(const PlanIn& p, int len) {
  return min(max(len, 0), p.width * kPage);
}
__device__ __forceinline__ int plan_row_len(const PlanIn& p, int r) {
  return plan_clamp(p, plan_row_raw(p, r));
}

constexpr int kPlanCachedTiles = 8;  // rows <= 512 keep their lengths in registers

struct PlanItem {
  int b, g, p0, p1, len;
  bool valid;
};

// The cached row lengths, in one round trip: straight-line loads at clamped
// rows (a load under a branch would be waited for on the spot).
__device__ __forceinline__ void plan_load(const PlanIn& p, int (&lenc)[kPlanCachedTiles]) {
  const int lane = threadIdx.x & 63;
  const int rows = p.B * p.Hkv;
#pragma unroll
  for (int t = 0; t < kPlanCachedTiles; ++t) lenc[t] = plan_row_raw(p, min(t * 64 + lane, rows - 1));
}

// The item plan_find gives when every row holds `width` pages (a full table,
// or a compact view filled to its capacity): the same closed form without a
// load.  A wave starts the loads of this item (query rows, table entries)
// while the row lengths are in flight, and keeps them when the plan agrees.
// Items per row when every row fills the table (0: the plan would not take
// its equal-rows form), and their chunk.
__device__ __forceinline__ int plan_full_rows(const PlanIn& p, int& chunk) {
  const int rows = p.B * p.Hkv;
  const int n = p.width;
  chunk = 0;
  if (p.target < rows || n <= 0) return 0;
  const int per_row = p.target / rows;
  chunk = max((n + per_row - 1) / per_row, kMinChunk);
  return (n + chunk - 1) / chunk;
}

__device__ __forceinline__ PlanItem plan_guess(const PlanIn& p, int item) {
  PlanItem it{0, 0, 0, 0, 0, false};
  const int rows = p.B * p.Hkv;
  const int n = p.width;
  int chunk;
  const int n_row = plan_full_rows(p, chunk);
  if (n_row == 0) return it;
  const int last_len = n - (n_row - 1) * chunk;
  const int shift = ((n_row & 1) == 0 && last_len > chunk / 40) ? chunk / 40 : 0;
  const int r = item / n_row;
  if (r >= rows) return it;
  const int j = item - r * n_row;
  it.b = r / p.Hkv;
  it.g = r % p.Hkv;
  it.p0 = j * chunk;
  it.p1 = min(n, it.p0 + chunk);
  if (j & 1) it.p0 += shift;
  else if (it.p1 < n) it.p1 += shift;
  it.valid = true;
  return it;
}

// One wave, over the lengths plan_load fetched.  If row_off is non-null, also
// publishes the per-row first item and the item count (done by work item 0
// for the merge kernel).
__device__ PlanItem plan_find(const PlanIn& p, int item, int32_t* row_off, int32_t* n_items,
                              int (&lenc)[kPlanCachedTiles]) {
  const int lane = threadIdx.x & 63;
  const int rows = p.B * p.Hkv;
  // total pages (< 2^28: rows <= 4096, width <= 65536) and the longest row
  int local = 0, longest = 0;
#pragma unroll
  for (int t = 0; t < kPlanCachedTiles; ++t) {
    lenc[t] = (t * 64 + lane >= rows) ? 0 : plan_clamp(p, lenc[t]);
    const int np = (lenc[t] + kPage - 1) / kPage;
    local += np;
    longest = max(longest, np);
  }
  for (int r = kPlanCachedTiles * 64 + lane; r < rows; r += 64) {
    const int np = (plan_row_len(p, r) + kPage - 1) / kPage;
    local += np;
    longest = max(longest, np);
  }
  local = wave_sum(local);
  longest = wave_max_nonneg(longest);
  // The chunk is the smallest with sum over rows of ceil(pages / chunk) <=
  // target, so that the plan fills one resident round without leaving a
  // wave's worth of slots empty.  When every row has the same length n (a
  // full table, or a pooled selection) that is ceil(n / floor(target / rows)).
  // Otherwise every row may end in a partial item, and total / (target -
  // rows) satisfies it (at least target / 2 as the divisor).
  int chunk;
  int shift = 0;  // pages moved from each odd item to the even item before it
  if (local == longest * rows && p.target >= rows && longest > 0) {
    const int per_row = p.target / rows;
    chunk = max((longest + per_row - 1) / per_row, kMinChunk);
    // Consecutive block ids go to consecutive XCDs, and on MI355X the waves
    // of the odd-numbered ones stream HBM about 5 % slower (per-wave
    // timelines, random page placement).  With an even item count per row,
    // item parity is block-id parity, so odd items give chunk / 40 pages to
    // the even item before them: the two halves then end together (measured:
    // chunk / 64 and chunk / 20 both gain less).  The last item (odd) keeps at
    // least one page.
    const int n_row = (longest + chunk - 1) / chunk;
    const int last_len = longest - (n_row - 1) * chunk;
    if ((n_row & 1) == 0 && last_len > chunk / 40) shift = chunk / 40;
  } else {
    const int aim = max(p.target - rows, max(p.target / 2, 1));
    chunk = max((local + aim - 1) / aim, kMinChunk);
    if (rows <= kPlanCachedTiles * 64) {
      // Ragged rows: that bound can leave the longest items far above the
      // average, and the call lasts as long as its longest items.  Search
      // for the smallest chunk whose items still fit the target, between the
      // even split and the bound (every wave computes the same value from
      // the cached lengths).
      int lo = max((local + p.target - 1) / p.target, kMinChunk), hi = chunk;
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        int n = 0;
#pragma unroll
        for (int t = 0; t < kPlanCachedTiles; ++t) n += ((lenc[t] + kPage - 1) / kPage + mid - 1) / mid;
        n = wave_sum(n);
        if (n <= p.target) hi = mid;
        else lo = mid + 1;
      }
      chunk = lo;
    }
  }
  PlanItem it{0, 0, 0, 0, 0, false};
  int carry = 0;
  for (int base = 0, t = 0; base < rows; base += 64, ++t) {
    const int r = base + lane;
    int ln = 0;
    if (t < kPlanCachedTiles) {
#pragma unroll
      for (int u = 0; u < kPlanCachedTiles; ++u)
        if (u == t) ln = lenc[u];
    } else if (r < rows) {
      ln = plan_row_len(p, r);
    }
    const int np = (ln + kPage - 1) / kPage;
    const int n = (np + chunk - 1) / chunk;
    const int incl = wave_incl_scan(n);
    const int excl = carry + incl - n;
    if (row_off && r < rows) row_off[r] = excl;
    const uint64_t hit = __ballot(r < rows && item >= excl && item < excl + n);
    if (hit && !it.valid) {
      const int src = __ffsll((unsigned long long)hit) - 1;  // wave-uniform
      const int rr = base + src;
      const int j = item - __builtin_amdgcn_readlane(excl, src);
      const int np_src = __builtin_amdgcn_readlane(np, src);
      it.b = rr / p.Hkv;
      it.g = rr % p.Hkv;
      it.p0 = j * chunk;
      it.p1 = min(np_src, it.p0 + chunk);
      if (j & 1) it.p0 += shift;
      else if (it.p1 < np_src) it.p1 += shift;
      it.len = __builtin_amdgcn_readlane(ln, src);
      it.valid = true;
    }
    carry += __builtin_amdgcn_readlane(incl, 63);
    if (it.valid && !row_off) break;
  }
  if (row_off && lane == 0) {
    row_off[rows] = carry;
    *n_items = carry;
  }
  return it;
}

// A wave-uniform value read with a vector load (every lane the same address),
// then moved to a scalar register.  The compiler moves scalar loads of
// read-only data down to their first use; these stay where they stand, so
// they are in flight together with the loads around them.
__device__ __forceinline__ int ld_uniform(const int32_t* p) {
  int z = 0;
  asm volatile("" : "+v"(z));  // an index the compiler cannot see is 0
  return p[z];
}

// Rotate one query element pair at position `pos`: (x, y) -> (x c - y s, y c + x s).
__device__ __forceinline__ float2 rope_pair(double x, double y, double s, double c) {
  return make_float2((float)(x * c - y * s), (float)(y * c + x * s));
}

struct PartArgs {
  const void* q;  // unrotated queries [B][q_len][Hq][D]
  const void* k;
  const void* v;
  const int32_t* table;
  const int32_t* logical;  // logical page of each table entry, or null: entry j is page j
  int32_t width, G;
  const int32_t* lens;
  const int32_t* pos;
  int32_t B;
  int32_t* row_off;
  int32_t* n_items;
  float* part_o;
  float2* part_ml;
  int32_t q_len, Hq, Hkv, grp, R;
  float scale_log2;
  double log2_theta;
  int32_t target;
};

// ------------------------------------------------------------------ bf16 MFMA partial
// NT row tiles of 16 query rows per wave (rows = GQA group x window, row r is
// query r / grp of head g*grp + r % grp).
//
// Memory pipeline, three disciplines (MODE selects), measured at 128K:
//  * throttled (long page runs, 16-row tiles): a four-page register ring whose
//    loads sit under branches, so each wave waits for every load in flight
//    before it computes and has about one page outstanding (page-table entries
//    fetched 64 at a time into one lane register each, broadcast with
//    readlane).  Two waves per SIMD hide each other's compute.
//  * staggered (long page runs, 32-row tiles): straight-line loads one page
//    ahead of the pair being consumed, so about one page stays in flight while
//    the single wave per SIMD computes.
//  * pairs (short items of a selected view, and 48/64-row tiles at any
//    length): straight-line loads of one pair at a time, requested as soon as
//    the previous pair is consumed; with one row tile and items of at least
//    eight pages, two pairs in flight (one consumed while the other arrives).
// The straight-line disciplines read page-table entries through scalar loads
// and make every page load unconditional, so the compiler waits for exactly
// the loads about to be consumed: the staggered loop clamps pages past the
// item to its last page (scores masked; at most two such loads per item), and
// the pair loop consumes its last pair after the loop and requests none.
// V is read with the non-temporal policy (each byte once per call) and K with
// the default one: each K fragment load covers half of a 128-byte line whose
// other half the next load takes, and early eviction between the two costs
// more than it saves.
// The query fragments live in LDS (re-read per pair) to keep the register
// footprint in budget: at D = 128, NT = 1 runs two waves per SIMD and
// NT = 2..4 one, with no spills.  NT = 3 and 4 let a (b, g) row group of up to
// 64 rows (e.g. a 5..8-token window under GQA 8:1) read each page once.
// Online softmax with a lazy reference max: a row's reference only moves
// when its running max exceeds it by more than 2^8 (log2 units), so the
// O rescale is skipped wave-wide on almost every pair; probabilities stay
// below 2^8, well inside bf16/fp32 range.  The final (m, l) pair uses the
// reference, so the merged result is the same softmax.
constexpr float kLazyRescale = 8.0f;

template <int D>
struct PageFrag {
  uint4 k[D / 32];
  uint2 v[D / 16];
  int lp;  // logical page (the causal mask compares logical positions)
};

// kPairs2: the pair loop with two pairs in flight (one row tile, items of at least eight pages)
enum { kThrottled = 0, kPairs = 1, kStaggered = 2, kPairs2 = 3 };

template <int D, int NT, int MODE>
__global__ __launch_bounds__(64, NT == 1 ? 2 : 1) void attn_partial_bf16(PartArgs a) {
  const PlanIn pin{a.lens, a.B, a.Hkv, a.G, a.width, a.target};
  const bool publish = blockIdx.x == 0 && blockIdx.y == 0;
  const int lane = threadIdx.x;
  const int l16 = lane & 15, q4 = lane >> 4;
  const int row0 = blockIdx.y * 16 * NT;
  constexpr int KS = D / 32;  // QK k-steps
  constexpr int NC = D / 16;  // PV dim tiles
  constexpr bool STRAIGHT = MODE != kThrottled;  // straight-line loads, scalar table reads
  constexpr bool PAIRS = MODE == kPairs || MODE == kPairs2;
  static_assert(MODE != kPairs2 || NT == 1, "two pairs in flight only with one row tile");
  constexpr int SR = 16 * NT;   // rows per slice
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  constexpr int QPL = SR * CPR / 64;  // chunks per lane
  // logical pages of the entries (a compact view), or none: entry p is page p
  const bool has_lg = a.logical != nullptr;
  // table row of (b, g), and its logical row (the table row itself, never
  // used, when there is none); a zero-width table has no entry to read, so
  // its reads are pointed at the lengths instead (never used either)
  const bool tab_ok = a.width > 0;
  auto trow_of = [&](int b, int g) -> const int32_t* {
    return tab_ok ? a.table + (int64_t)(b * a.G + (a.G == 1 ? 0 : g)) * a.width : a.lens;
  };
  auto lrow_of = [&](int b, int g) -> const int32_t* {
    return (has_lg && tab_ok) ? a.logical + (int64_t)(b * a.G + (a.G == 1 ? 0 : g)) * a.width
                              : trow_of(b, g);
  };
  // The straight-line modes read the (read-only) tables through the constant address
  // space: the wave-uniform entries then come through scalar memory and its
  // own counter, so waiting for an entry never waits for K/V loads in flight.
  auto as_const = [](const int32_t* p) { return (const __attribute__((address_space(4))) int32_t*)p; };

  // This slice's query rows of (b, g): rows past R load row R - 1 and are
  // masked to zero (straight-line: a load under a branch would be waited for
  // on the spot).
  uint4 qraw[QPL];
  auto load_q = [&](int b, int g) {
    const uint16_t* q = (const uint16_t*)a.q;
#pragma unroll
    for (int k = 0; k < QPL; ++k) {
      const int e = k * 64 + lane;
      const int rr = e / CPR, c = e % CPR;
      const int r = row0 + rr;
      const int rc = min(r, a.R - 1);
      const int i = rc / a.grp, h = g * a.grp + rc % a.grp;
      const uint4 x = *(const uint4*)(q + (((int64_t)b * a.q_len + i) * a.Hq + h) * D + 8 * c);
      const uint32_t keep = (r < a.R) ? 0xffffffffu : 0u;
      qraw[k] = make_uint4(x.x & keep, x.y & keep, x.z & keep, x.w & keep);
    }
  };
  // First table entries of an item [p0, p1): the pair's two entries and their
  // logical pages as scalars (straight-line modes), or the 64-entry window in
  // one lane register each (ring).
  int e0 = 0, e1 = 0, lg0 = 0, lg1 = 0, tr = 0, tl = 0;
  auto load_entries = [&](int b, int g, int p0, int p1, bool early) {
    const int32_t* tq = trow_of(b, g);
    const int32_t* lq = lrow_of(b, g);
    if constexpr (STRAIGHT) {
      const int f0 = tab_ok ? p0 : 0, f1 = tab_ok ? min(p0 + 1, p1 - 1) : 0;
      if (early) {  // issued ahead of the plan: vector loads stay where they stand
        e0 = ld_uniform(tq + f0);
        e1 = ld_uniform(tq + f1);
        const int x0 = ld_uniform(lq + f0), x1 = ld_uniform(lq + f1);
        lg0 = has_lg ? x0 : f0;
        lg1 = has_lg ? x1 : f1;
      } else {
        e0 = as_const(tq)[f0];
        e1 = as_const(tq)[f1];
        const int x0 = as_const(lq)[f0], x1 = as_const(lq)[f1];
        lg0 = has_lg ? x0 : f0;
        lg1 = has_lg ? x1 : f1;
      }
    } else {
      const int f = tab_ok ? min(p0 + lane, p1 - 1) : 0;  // entries past the item are never used
      tr = tq[f];
      const int x = lq[f];
      tl = has_lg ? x : 0;
    }
  };

  // Start.  For long items (the throttled ring and the staggered loop: full
  // tables, verify windows) the loads of the item the plan gives when every
  // row fills the table (plan_guess) -- its query rows, position and first
  // table entries -- go out first, then the row lengths for the plan itself,
  // all in one round trip (waiting for the lengths then waits for nothing
  // issued later).  When the plan agrees, the guessed loads are kept;
  // otherwise they are made again for the real item.  Page loads wait for the
  // plan: a table entry past a row's end may be -1.  Measured on the 128K
  // verify: its first pages are consumed 2.3 us earlier (340 against 342 us
  // per call).  The pair loop of short items (a selected view) keeps the
  // plan-first order, which measured 0.4 us faster there: a burst of start-up
  // loads from every wave at once returns later than the same loads issued
  // after the plan.
  constexpr bool SPECULATE = !PAIRS;
  PlanItem sp{0, 0, 0, 0, 0, false};
  if constexpr (SPECULATE) sp = plan_guess(pin, blockIdx.x);
  const int sb = sp.valid ? sp.b : 0, sg = sp.valid ? sp.g : 0;
  const int sp0 = sp.valid ? sp.p0 : 0, sp1 = sp.valid ? sp.p1 : 1;
  int pos_b = 0;
  if constexpr (SPECULATE) {
    load_q(sb, sg);
    pos_b = ld_uniform(a.pos + sb);
    load_entries(sb, sg, sp0, sp1, true);
  }
  int lenc[kPlanCachedTiles];
  plan_load(pin, lenc);
  // every load above is issued before the first wait (the scheduler would
  // otherwise start the plan's waits between them)
  asm volatile("" ::: "memory");
  const PlanItem it = plan_find(pin, blockIdx.x, publish ? a.row_off : nullptr, a.n_items, lenc);
  if (!it.valid) return;
  const int item = blockIdx.x;
  // the item is the same for every lane: keep it in scalar registers
  const int b = __builtin_amdgcn_readfirstlane(it.b), g = __builtin_amdgcn_readfirstlane(it.g);
  const int p0 = __builtin_amdgcn_readfirstlane(it.p0), p1 = __builtin_amdgcn_readfirstlane(it.p1);
  const int len = __builtin_amdgcn_readfirstlane(it.len);
  if (!(sp.valid && sb == b && sg == g && sp0 == p0 && sp1 == p1)) {
    // no guess, or rows shorter than the table (wave-uniform)
    // The position comes through the constant space like the table entries:
    // as a plain load the compiler makes it a vector load (the kernel's own
    // stores keep it from proving the array read-only), and moving it to a
    // scalar register then waits for every vector load before it (the query
    // rows), which held the table entries, and so the first pages, back by
    // one round trip (selected decode at 128K: 29.8-29.9 -> 29.0-29.1 us).
    load_q(b, g);
    pos_b = SPECULATE ? ld_uniform(a.pos + b) : as_const(a.pos)[b];
    load_entries(b, g, p0, p1, false);
  }
  pos_b = __builtin_amdgcn_readfirstlane(pos_b);
  const int32_t* trow = trow_of(b, g);
  const int32_t* lrow = lrow_of(b, g);
  const auto trow_s = as_const(trow);
  const auto lrow_s = as_const(lrow);
  const uint16_t* kpool = (const uint16_t*)a.k;
  const uint16_t* vpool = (const uint16_t*)a.v;
  const int64_t head_off = (int64_t)g * (kPage * D);
  const int64_t page_stride = (int64_t)a.Hkv * (kPage * D);
  const int k_lane = l16 * D + 8 * q4;
  const int v_lane = l16 * kPage + 4 * q4;

  // page-table window of the ring: lane j holds trow[wbase + j] (and its logical page)
  int wbase = p0;
  auto phys_of = [&](int p) -> int64_t {
    if constexpr (STRAIGHT) {
      return (int64_t)trow_s[p];
    } else {
      if (p - wbase >= 64) {  // wave-uniform refill
        wbase += 64;
        tr = trow[min(wbase + lane, p1 - 1)];
        if (has_lg) tl = lrow[min(wbase + lane, p1 - 1)];
      }
      return (int64_t)__builtin_amdgcn_readlane(tr, p - wbase);
    }
  };
  // logical page of entry p; for the ring, after phys_of(p) has set the window
  auto logical_of = [&](int p) -> int {
    if (!has_lg) return p;
    if constexpr (STRAIGHT) return lrow_s[p];
    else return __builtin_amdgcn_readlane(tl, p - wbase);
  };
  auto load_at = [&](int64_t phys, int lp, PageFrag<D>& f) {
    const int64_t base = phys * page_stride + head_off;
    f.lp = lp;
    const uint16_t* kp = kpool + base + k_lane;
    const uint16_t* vp = vpool + base + v_lane;
#pragma unroll
    for (int s = 0; s < KS; ++s) f.k[s] = *(const uint4*)(kp + 32 * s);
#pragma unroll
    for (int c = 0; c < NC; ++c)
      f.v[c] = ld_stream8(vp + 16 * kPage * c);
  };
  auto load_page = [&](int p, PageFrag<D>& f) {
    const int64_t phys = phys_of(p);
    load_at(phys, logical_of(p), f);
  };

  // page buffers: the throttled ring and the staggered loop use four, the
  // pair loop two
  PageFrag<D> buf0, buf1, buf2, buf3;
#pragma unroll
  for (int s = 0; s < KS; ++s) buf0.k[s] = buf1.k[s] = buf2.k[s] = buf3.k[s] = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int c = 0; c < NC; ++c) buf0.v[c] = buf1.v[c] = buf2.v[c] = buf3.v[c] = make_uint2(0, 0);
  buf0.lp = buf1.lp = buf2.lp = buf3.lp = 0;
  if constexpr (STRAIGHT) {
    // straight-line: the first pair, from the entries read at the start (the
    // staggered loop requests the next page itself before consuming it)
    load_at(__builtin_amdgcn_readfirstlane(e0), lg0, buf0);
    load_at(__builtin_amdgcn_readfirstlane(e1), lg1, buf1);
    // two pairs in flight: the second pair goes out here too (clamped into
    // the item, which has at least eight pages on this path's calls; a
    // shorter one reads its last page again)
    if constexpr (MODE == kPairs2) {
      load_page(min(p0 + 2, p1 - 1), buf2);
      load_page(min(p0 + 3, p1 - 1), buf3);
    }
  } else {
    // the first four pages go out together (straight-line, past the item
    // clamped to its last page: never consumed unmasked; their table entries
    // read straight from the window, which holds them), so they arrive in
    // one round trip and the query rotation below runs while they are in
    // flight; the main loop then throttles to about one page per wave
    auto load_first = [&](int k, PageFrag<D>& f) {
      const int p = min(p0 + k, p1 - 1);
      load_at((int64_t)__builtin_amdgcn_readlane(tr, p - p0),
              has_lg ? __builtin_amdgcn_readlane(tl, p - p0) : p, f);
    };
    load_first(0, buf0);
    load_first(1, buf1);
    load_first(2, buf2);
    load_first(3, buf3);
  }

  // This slice's query rows, rotated at their positions, as LDS fragments in
  // the B-operand layout of S^T = K Q^T (row l16, dims 32 s + 8 q4 .. + 7).
  __shared__ uint16_t sraw[SR][D];
  __shared__ uint4 sq[NT][KS][64];
  int qpos[NT];
  {
#pragma unroll
    for (int k = 0; k < QPL; ++k) {
      const int e = k * 64 + lane;
      *(uint4*)&sraw[e / CPR][8 * (e % CPR)] = qraw[k];
    }
    lds_barrier();  // LDS only: the first pages stay in flight
    constexpr int HALF = D / 2, LPP = 64 / HALF;
    const int pr = lane % HALF, rsub = lane / HALF;
    uint16_t* sqh = (uint16_t*)&sq[0][0][0];
    auto frag_at = [&](int rr, int dim) {
      return ((((rr >> 4) * KS + (dim >> 5)) * 64) + (rr & 15) + 16 * ((dim & 31) >> 3)) * 8 +
             (dim & 7);
    };
    // Rows r of query i = r / grp share one angle: one fp64 sincos at the
    // slice's first position and, for a window, one of the per-position step,
    // then each next position by fp64 angle addition (it agrees with a direct
    // sincos to about 1e-16, far below the bf16 rounding of the rotated rows;
    // 4-token verify 337.9-338.7 -> 337.5-337.9 us), then the rows of that
    // position.  The
    // fragment offset of (row rr, dim) is frag_at(0, dim) plus a row term, so
    // each lane's two offsets are computed once; both halves are rounded by
    // one conversion instruction.  Rows past R are written as zeros.
    const int fx = frag_at(0, pr), fy = frag_at(0, pr + HALF);
    auto row_term = [](int rr) { return (rr >> 4) * (KS * 512) + (rr & 15) * 8; };
    const int rq = min(SR, a.R - row0);  // rows of this slice that hold queries
    const int i_lo = row0 / a.grp, i_hi = (row0 + rq - 1) / a.grp;
    double sn, cs, s1 = 0.0, c1 = 1.0;
    rope_sincos((double)pos_b + (double)i_lo, pr, D, a.log2_theta, &sn, &cs);
    if (i_hi > i_lo) rope_step(pr, D, a.log2_theta, &s1, &c1);  // uniform
    for (int i = i_lo; i <= i_hi; ++i) {
      if (i > i_lo) {  // the next position by angle addition (fp64)
        const double ns = fma(sn, c1, cs * s1), nc = fma(cs, c1, -(sn * s1));
        sn = ns;
        cs = nc;
      }
      const int ra = max(i * a.grp - row0, 0);
      const int rb = min((i + 1) * a.grp - row0, rq);
#pragma unroll 4
      for (int rr = ra + rsub; rr < rb; rr += LPP) {
        const float2 v = rope_pair(bf16_to_f32(sraw[rr][pr]), bf16_to_f32(sraw[rr][pr + HALF]), sn, cs);
        const uint32_t h = pack_bf16x2(v.x, v.y);
        sqh[fx + row_term(rr)] = (uint16_t)h;
        sqh[fy + row_term(rr)] = (uint16_t)(h >> 16);
      }
    }
    for (int rr = rq + rsub; rr < SR; rr += LPP) {
      sqh[fx + row_term(rr)] = 0;
      sqh[fy + row_term(rr)] = 0;
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int r = row0 + 16 * t + l16;
      qpos[t] = (r < a.R) ? pos_b + r / a.grp : -1;
    }
    lds_barrier();
  }

  floatx4 o[NT][NC];
  float m[NT], l[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    m[t] = -INFINITY;
    l[t] = 0.f;
#pragma unroll
    for (int c = 0; c < NC; ++c) o[t][c] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  // Invisible slots of a partial last page may hold anything: zero their V.
  auto mask_v = [&](int p, PageFrag<D>& f) {
    const int nvalid = len - p * kPage;
    if (nvalid < kPage) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        uint32_t lo = f.v[c].x, hi = f.v[c].y;
        const int j0 = 4 * q4;
        if (j0 + 0 >= nvalid) lo &= 0xffff0000u;
        if (j0 + 1 >= nvalid) lo &= 0x0000ffffu;
        if (j0 + 2 >= nvalid) hi &= 0xffff0000u;
        if (j0 + 3 >= nvalid) hi &= 0x0000ffffu;
        f.v[c] = make_uint2(lo, hi);
      }
    }
  };

  // One pair of pages (p, p + 1).  S^T for each page on 16x16x32 MFMAs; one
  // softmax reference per pair; then O^T += V^T P^T over the pair's 32 tokens
  // on 16x16x32 MFMAs, with contraction index 8 q4 + e standing for token
  // 4 q4 + e of page p (e < 4) or 4 q4 + e - 4 of page p + 1 (e >= 4): the
  // lane's V^T operand is its two 8-byte V loads side by side, its P^T operand
  // its two groups of 4 probabilities.  When page p + 1 is not part of the
  // item (hb false) its scores are masked and its buffer holds finite values
  // (zeros or an earlier, already masked page), so it adds nothing.
  auto consume2 = [&](int p, PageFrag<D>& fa, PageFrag<D>& fb, bool hb) {
    mask_v(p, fa);
    mask_v(p + 1, fb);
    // re-read the query fragments from LDS every pair (an opaque index keeps
    // the compiler from hoisting them into registers)
    int ql = lane;
    asm volatile("" : "+v"(ql));
    // The NT row tiles are independent: each stage runs across all tiles
    // before the next, so one tile's MFMA latency hides behind another's
    // VALU work, and one wave-wide vote decides the rare reference move.
    floatx4 sa[NT], sb[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      sa[t] = floatx4{0.f, 0.f, 0.f, 0.f};
      sb[t] = floatx4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int s = 0; s < KS; ++s)
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const bf16x8 qf = __builtin_bit_cast(bf16x8, sq[t][s][ql]);
        sa[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fa.k[s]), qf,
                                                       sa[t], 0, 0, 0);
        sb[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, fb.k[s]), qf,
                                                       sb[t], 0, 0, 0);
      }
    // length test on the entry index, causal test on the logical position
    const int tok0 = p * kPage + 4 * q4;
    const int la0 = fa.lp * kPage + 4 * q4, lb0 = fb.lp * kPage + 4 * q4;
    float za[NT][4], zb[NT][4], mx[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      mx[t] = -INFINITY;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int ta = tok0 + j, tb = tok0 + kPage + j;
        za[t][j] = (ta < len && la0 + j <= qpos[t]) ? sa[t][j] * a.scale_log2 : -INFINITY;
        zb[t][j] = (hb && tb < len && lb0 + j <= qpos[t]) ? sb[t][j] * a.scale_log2 : -INFINITY;
        mx[t] = fmaxf(mx[t], fmaxf(za[t][j], zb[t][j]));
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) mx[t] = rows_max(mx[t]);
    // move a row's reference only when its running max clears it by kLazyRescale
    bool bump[NT];
    bool any = false;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      bump[t] = mx[t] > m[t] + kLazyRescale || (m[t] == -INFINITY && mx[t] != -INFINITY);
      any = any || bump[t];
    }
    if (__ballot(any)) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const float mn = bump[t] ? mx[t] : m[t];  // unmoved rows scale by exp2(0) = 1
        const float alpha = (m[t] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(m[t] - mn);
        l[t] *= alpha;
#pragma unroll
        for (int c = 0; c < NC; ++c) o[t][c] *= alpha;
        m[t] = mn;
      }
    }
    bf16x8 pf[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      float pa[4], pb[4];
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        pa[j] = (za[t][j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(za[t][j] - m[t]);
        pb[j] = (zb[t][j] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(zb[t][j] - m[t]);
        psum += pa[j] + pb[j];
      }
      l[t] += psum;
      pf[t] = __builtin_bit_cast(bf16x8, make_uint4(pack_bf16x2(pa[0], pa[1]), pack_bf16x2(pa[2], pa[3]),
                                                    pack_bf16x2(pb[0], pb[1]), pack_bf16x2(pb[2], pb[3])));
    }
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      // the two pages' 8-byte V loads side by side (as native vectors: kept in registers)
      const bf16x8 vf = __builtin_bit_cast(
          bf16x8, __builtin_shufflevector(__builtin_bit_cast(u32x2v, fa.v[c]),
                                          __builtin_bit_cast(u32x2v, fb.v[c]), 0, 1, 2, 3));
#pragma unroll
      for (int t = 0; t < NT; ++t)
        o[t][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[t], o[t][c], 0, 0, 0);
    }
  };

  if constexpr (MODE == kStaggered) {
    // one page ahead: while a pair is consumed, the first page of the next
    // pair is in flight, and its second page is requested right after
    for (int p = p0; p < p1; p += 4) {
      load_page(min(p + 2, p1 - 1), buf2);
      consume2(p, buf0, buf1, p + 1 < p1);
      load_page(min(p + 3, p1 - 1), buf3);
      if (p + 2 >= p1) break;
      load_page(min(p + 4, p1 - 1), buf0);
      consume2(p + 2, buf2, buf3, p + 3 < p1);
      load_page(min(p + 5, p1 - 1), buf1);
    }
  } else if constexpr (PAIRS) {
    if constexpr (MODE == kPairs2) {
      // Two pairs in flight: A = (p, p + 1) and B = (p + 2, p + 3) went out
      // in the prologue (clamped into the item); while one pair is consumed
      // the other is in flight, and each is refilled right after it is
      // consumed.  Inside the loop every load is unconditional, so the
      // compiler waits for exactly the pair about to be consumed; the last
      // one to seven pages are consumed after it, the pages past the first
      // four a pair at a time, so no page past the item is requested (clamped
      // copies would be fetched again: V streams).
      int p = p0;
      for (; p + 8 <= p1; p += 4) {
        consume2(p, buf0, buf1, true);
        load_page(p + 4, buf0);
        load_page(p + 5, buf1);
        consume2(p + 2, buf2, buf3, true);
        load_page(p + 6, buf2);
        load_page(p + 7, buf3);
      }
      // pages left: 1..7 (uniform); A and B hold the next four (clamped)
      const int r = p1 - p;
      consume2(p, buf0, buf1, r >= 2);
      if (r >= 3) consume2(p + 2, buf2, buf3, r >= 4);
      for (int q = p + 4; q < p1; q += 2) {  // at most two more pairs, one at a time
        load_page(q, buf0);
        load_page(min(q + 1, p1 - 1), buf1);
        consume2(q, buf0, buf1, q + 1 < p1);
      }
    } else {
      // one pair in flight; the last pair is consumed after the loop, so no
      // pages past the item are requested
      int p = p0;
      for (; p + 2 < p1; p += 2) {
        consume2(p, buf0, buf1, true);
        load_page(p + 2, buf0);
        load_page(min(p + 3, p1 - 1), buf1);
      }
      consume2(p, buf0, buf1, p + 1 < p1);
    }
  } else {
    for (int p = p0; p < p1; p += 4) {
      consume2(p, buf0, buf1, p + 1 < p1);
      if (p + 4 < p1) load_page(p + 4, buf0);
      if (p + 5 < p1) load_page(p + 5, buf1);
      if (p + 2 < p1) {
        consume2(p + 2, buf2, buf3, p + 3 < p1);
        if (p + 6 < p1) load_page(p + 6, buf2);
        if (p + 7 < p1) load_page(p + 7, buf3);
      }
    }
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    l[t] = rows_sum(l[t]);
    const int r = row0 + 16 * t + l16;
    if (r < a.R) {
      // The partial output normalized by its own sum, in bf16 (the sum and
      // the reference max stay fp32): half the bytes the merge reads back,
      // with the range of fp32.  Against the fp64 oracle the largest row
      // error at full size went from 1.30-2.02e-3 to 1.50-2.10e-3 (bf16
      // output, tolerance 2e-2); step 33.27-33.28K -> 33.55-33.64K tokens/s
      // (verify -2 us, selected decode -0.6 us).  fp16 measured as fast and
      // as accurate as fp32 partials, but overflows past 65504.
      const float inv = l[t] > 0.f ? 1.f / l[t] : 0.f;
      uint16_t* dst = (uint16_t*)a.part_o + ((int64_t)item * a.R + r) * D + 4 * q4;
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const floatx4 v = o[t][c] * inv;
        *(uint2*)(dst + 16 * c) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
      if (q4 == 0) a.part_ml[(int64_t)item * a.R + r] = make_float2(m[t], l[t]);
    }
  }
}

// ------------------------------------------------------------------ fp32 VALU partial
// One wave per (item, slice of up to 32 rows).  Page tiles staged in LDS; each
// lane owns (row, token) score pairs, then (row, dim) output pairs.
template <int D>
__global__ __launch_bounds__(64) void attn_partial_f32(PartArgs a) {
  const PlanIn pin{a.lens, a.B, a.Hkv, a.G, a.width, a.target};
  const bool publish = blockIdx.x == 0 && blockIdx.y == 0;
  int lenc[kPlanCachedTiles];
  plan_load(pin, lenc);
  const PlanItem it = plan_find(pin, blockIdx.x, publish ? a.row_off : nullptr, a.n_items, lenc);
  if (!it.valid) return;
  const int item = blockIdx.x;
  const int b = it.b, g = it.g, p0 = it.p0, p1 = it.p1;
  const int lane = threadIdx.x;
  constexpr int RS = 32;                 // rows per slice
  const int row0 = blockIdx.y * RS;
  const int nr = min(RS, a.R - row0);
  const int gr = a.G == 1 ? 0 : g;
  const int len = it.len;
  const int32_t* trow = a.table + (int64_t)(b * a.G + gr) * a.width;
  const float* qin = (const float*)a.q;
  const float* kpool = (const float*)a.k;
  const float* vpool = (const float*)a.v;

  __shared__ float sq[RS][D];
  __shared__ float sk[kPage][D + 1];
  __shared__ float sv[D][kPage + 1];
  __shared__ float sp[RS][kPage];
  __shared__ float s_alpha[RS];
  __shared__ int s_qpos[RS];
  // rotate this slice's query rows (fp64 angles) straight into LDS
  constexpr int HALF = D / 2;
  for (int e = lane; e < nr * HALF; e += 64) {
    const int rr = e / HALF, pr = e % HALF;
    const int r = row0 + rr;
    const int i = r / a.grp, h = g * a.grp + r % a.grp;
    double sn, cs;
    rope_sincos((double)a.pos[b] + (double)i, pr, D, a.log2_theta, &sn, &cs);
    const float* src = qin + (((int64_t)b * a.q_len + i) * a.Hq + h) * D;
    const float2 v = rope_pair(src[pr], src[pr + HALF], sn, cs);
    sq[rr][pr] = v.x;
    sq[rr][pr + HALF] = v.y;
  }
  if (lane < nr) s_qpos[lane] = a.pos[b] + (row0 + lane) / a.grp;
  constexpr int DPL = (D + 63) / 64;     // dims per lane
  float acc[RS][DPL];
  float mrow = -INFINITY, lrow = 0.f;    // lane r < nr keeps row r's running stats
#pragma unroll
  for (int rr = 0; rr < RS; ++rr)
#pragma unroll
    for (int u = 0; u < DPL; ++u) acc[rr][u] = 0.f;
  __syncthreads();
  const int32_t* ltab = a.logical ? a.logical + (int64_t)(b * a.G + gr) * a.width : nullptr;
  for (int p = p0; p < p1; ++p) {
    const int64_t phys = trow[p];
    const int lpos0 = (ltab ? ltab[p] : p) * kPage;  // logical position of the page's slot 0
    const float* kp = kpool + (phys * a.Hkv + g) * (int64_t)(kPage * D);
    const float* vp = vpool + (phys * a.Hkv + g) * (int64_t)(D * kPage);
    const int nvalid = min(kPage, len - p * kPage);
    for (int e = lane; e < kPage * D; e += 64) {
      const int t = e / D, d = e % D;
      sk[t][d] = kp[e];
      const int dv = e / kPage, tv = e % kPage;
      const float vv = vp[e];
      sv[dv][tv] = (tv < nvalid) ? vv : 0.f;
    }
    __syncthreads();
    for (int e = lane; e < nr * kPage; e += 64) {
      const int rr = e / kPage, t = e % kPage;
      const int tok = p * kPage + t;
      float z = -INFINITY;
      if (tok < len && lpos0 + t <= s_qpos[rr]) {
        float dot = 0.f;
        for (int d = 0; d < D; ++d) dot += sq[rr][d] * sk[t][d];
        z = dot * a.scale_log2;
      }
      sp[rr][t] = z;
    }
    __syncthreads();
    if (lane < nr) {
      float mx = -INFINITY;
      for (int t = 0; t < kPage; ++t) mx = fmaxf(mx, sp[lane][t]);
      const float mn = fmaxf(mrow, mx);
      const float alpha = (mn == -INFINITY) ? 1.f : exp2f(mrow - mn);
      float ps = 0.f;
      for (int t = 0; t < kPage; ++t) {
        const float z = sp[lane][t];
        const float pz = (z == -INFINITY) ? 0.f : exp2f(z - mn);
        sp[lane][t] = pz;
        ps += pz;
      }
      lrow = lrow * alpha + ps;
      mrow = mn;
      s_alpha[lane] = alpha;
    }
    __syncthreads();
#pragma unroll
    for (int rr = 0; rr < RS; ++rr) {
      if (rr < nr) {
        const float al = s_alpha[rr];
#pragma unroll
        for (int u = 0; u < DPL; ++u) {
          const int d = lane + 64 * u;
          if (d < D) {
            float s = acc[rr][u] * al;
            for (int t = 0; t < kPage; ++t) s += sp[rr][t] * sv[d][t];
            acc[rr][u] = s;
          }
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int rr = 0; rr < RS; ++rr) {
    if (rr < nr) {
      const int r = row0 + rr;
      float* dst = a.part_o + ((int64_t)item * a.R + r) * D;
#pragma unroll
      for (int u = 0; u < DPL; ++u) {
        const int d = lane + 64 * u;
        if (d < D) dst[d] = acc[rr][u];
      }
    }
  }
  if (lane < nr) a.part_ml[(int64_t)item * a.R + row0 + lane] = make_float2(mrow, lrow);
}

struct MergeArgs {
  const int32_t* row_off;
  const float* part_o;
  const float2* part_ml;
  void* out;
  float* lse;
  int32_t out_dt;
  int32_t q_len, Hq, Hkv, grp, R;
};

// ------------------------------------------------------------------ merge
// Block (b, g, query row r): IG item groups x D/4 threads (4 dims each).  Each
// item group folds the items j = i0 + ig, i0 + ig + IG, ... in one pass with a
// running max (weights e^(m_j - M) rescaled as M grows); the groups are then
// combined in group order through LDS, so the result does not depend on
// scheduling.  PH: the partial outputs are bf16 and normalized by their own
// sums (the MFMA kernel's), so an item's output enters with weight
// e^(m_j - M) l_j; otherwise fp32 and unnormalized (the fp32 kernel's).
template <int D, bool PH>
__global__ __launch_bounds__(256) void attn_merge_kernel(MergeArgs a) {
  constexpr int TPR = D / 4, IG = 256 / TPR;
  const int bg = blockIdx.x, r = blockIdx.y;
  const int b = bg / a.Hkv, g = bg % a.Hkv;
  const int tid = threadIdx.x, ig = tid / TPR, t4 = tid % TPR, d4 = t4 * 4;
  const int i0 = a.row_off[bg], i1 = a.row_off[bg + 1];
  __shared__ float s_m[IG], s_l[IG];
  __shared__ floatx4 s_o[IG][TPR];
  float M = -INFINITY, L = 0.f;
  floatx4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 4
  for (int j = i0 + ig; j < i1; j += IG) {
    const float2 ml = a.part_ml[(int64_t)j * a.R + r];
    floatx4 o;
    if constexpr (PH) {
      const uint2 h = *(const uint2*)((const uint16_t*)a.part_o + ((int64_t)j * a.R + r) * D + d4);
      o = floatx4{__uint_as_float(h.x << 16), __uint_as_float(h.x & 0xffff0000u),
                  __uint_as_float(h.y << 16), __uint_as_float(h.y & 0xffff0000u)};
    } else {
      o = *(const floatx4*)(a.part_o + ((int64_t)j * a.R + r) * D + d4);
    }
    const bool seen = ml.x != -INFINITY;  // an item that saw no key adds nothing
    const float Mn = seen ? fmaxf(M, ml.x) : M;
    const float sc = (M == -INFINITY) ? 0.f : exp2f(M - Mn);
    const float w = seen ? exp2f(ml.x - Mn) : 0.f;
    L = L * sc + w * ml.y;
    O = O * sc + (PH ? w * ml.y : w) * o;
    M = Mn;
  }
  if (t4 == 0) {
    s_m[ig] = M;
    s_l[ig] = L;
  }
  s_o[ig][t4] = O;
  __syncthreads();
  if (ig != 0) return;
  M = -INFINITY;
#pragma unroll
  for (int k = 0; k < IG; ++k) M = fmaxf(M, s_m[k]);
  L = 0.f;
  O = floatx4{0.f, 0.f, 0.f, 0.f};
  if (M != -INFINITY) {
#pragma unroll
    for (int k = 0; k < IG; ++k) {
      const float w = exp2f(s_m[k] - M);  // 0 for groups that saw no key
      L += w * s_l[k];
      O += w * s_o[k][t4];
    }
  }
  const int i = r / a.grp, h = g * a.grp + r % a.grp;
  const int64_t orow = ((int64_t)b * a.q_len + i) * a.Hq + h;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  if (a.out_dt == KAP_BF16) {
    *(uint2*)((uint16_t*)a.out + orow * D + d4) =
        make_uint2(pack_bf16x2(O[0] * inv, O[1] * inv), pack_bf16x2(O[2] * inv, O[3] * inv));
  } else {
    *(floatx4*)((float*)a.out + orow * D + d4) = O * inv;
  }
  if (d4 == 0 && a.lse)
    a.lse[orow] = L > 0.f ? (M + log2f(L)) * 0.69314718055994531f : -INFINITY;
}

// ------------------------------------------------------------------ launcher
kap_status launch_attention(const AttnCall& c) {
  const int grp = c.Hq / c.Hkv;
  const int R = grp * c.q_len;
  PartArgs a{};
  a.q = c.q;
  a.k = c.k;
  a.v = c.v;
  a.table = c.table;
  a.logical = c.logical;
  a.width = c.width;
  a.G = c.G;
  a.lens = c.lens;
  a.pos = c.positions;
  a.B = c.B;
  a.row_off = c.ws.row_off;
  a.n_items = c.ws.n_items;
  a.part_o = c.ws.part_o;
  a.part_ml = c.ws.part_ml;
  a.q_len = c.q_len;
  a.Hq = c.Hq;
  a.Hkv = c.Hkv;
  a.grp = grp;
  a.R = R;
  a.scale_log2 = c.scale * 1.4426950408889634f;
  a.log2_theta = log2((double)c.theta);
  const void* fn;
  int slices;
  int item_cap = kTargetItems;
  if (c.dtype == KAP_BF16) {
    // one row slice whenever the rows fit in 64, so each page is read once per (b, g)
    const int nt = R <= 16 ? 1 : R <= 32 ? 2 : R <= 48 ? 3 : 4;
    slices = (R + 16 * nt - 1) / (16 * nt);
#define KAP_PARTIALS(D, M)                                                            \
  {(const void*)attn_partial_bf16<D, 1, M>, (const void*)attn_partial_bf16<D, 2, M>,      \
   (const void*)attn_partial_bf16<D, 3, M>, (const void*)attn_partial_bf16<D, 4, M>}
    static const void* const fns[4][2][4] = {
        {KAP_PARTIALS(64, kThrottled), KAP_PARTIALS(128, kThrottled)},
        {KAP_PARTIALS(64, kPairs), KAP_PARTIALS(128, kPairs)},
        {KAP_PARTIALS(64, kStaggered), KAP_PARTIALS(128, kStaggered)},
        {{(const void*)attn_partial_bf16<64, 1, kPairs2>, nullptr, nullptr, nullptr},
         {(const void*)attn_partial_bf16<128, 1, kPairs2>, nullptr, nullptr, nullptr}}};
#undef KAP_PARTIALS
    const int di = c.D == 128 ? 1 : 0;
    // Short work items (a selected view) are latency-bound, and the 48/64-row
    // tiles need their per-page compute to overlap the next pair's loads: both
    // run the pair loop.  Long items saturate HBM, where about one page in
    // flight per wave measured fastest: with 16-row tiles (two waves per SIMD)
    // the throttled ring, with 32-row tiles (one wave per SIMD, so nothing else
    // hides its compute) the staggered loop.  The host bounds the item length
    // from the table width, mirroring the device plan's chunk formula.
    const int rows = c.B * c.Hkv;
    const int t0 = max(1, min(kTargetItems, resident_blocks(fns[0][di][nt - 1], 64) / slices));
    const int aim = max(t0 - rows, max(t0 / 2, 1));
    const long long chunk = max(((long long)c.width * rows + aim - 1) / aim, (long long)kMinChunk);
    // (items of at least eight pages with one row tile keep two pairs in
    // flight: 12-page items of a 451-page view 32.9-33.1 -> 32.2-32.5 us;
    // 6-page items measured slower that way, 20.7-20.9 -> 21.6 us)
    int mode = (chunk <= kShortItemPages || nt >= 3)
                   ? (nt == 1 && chunk >= kPairs2MinPages ? kPairs2 : kPairs)
                   : nt == 1 ? kThrottled : kStaggered;
    // Items of four to seven pages are made eight long instead (fewer items,
    // capped so that a row of the table's width splits into eight-page
    // items) and run with two pairs in flight: two round trips per item
    // instead of three or four.  113-page views of 64 rows (Llama-shaped
    // 32K, B = 8): 1216 items of 6 pages 20.2 us -> 960 items of 8 pages
    // 19.8 us; views of 1 to 3 pages per item keep their many short items.
    if (mode == kPairs && nt == 1 && chunk >= 4 && c.width >= kPairs2MinPages) {
      item_cap = rows * ((c.width + kPairs2MinPages - 1) / kPairs2MinPages);
      mode = kPairs2;
    }
    fn = fns[mode][di][nt - 1];
  } else {
    slices = (R + 31) / 32;
    fn = c.D == 128 ? (const void*)attn_partial_f32<128> : (const void*)attn_partial_f32<64>;
  }
  // one round of resident waves, shared among the row slices
  a.target = max(1, min(item_cap, resident_blocks(fn, 64) / slices));
  void* args[] = {&a};
  const int max_items = a.target + c.B * c.Hkv;  // the plan never makes more
  const hipError_t e = hipLaunchKernel(fn, dim3(max_items, slices), dim3(64), args, 0, c.stream);
  if (e != hipSuccess) return fail(KAP_ERR_HIP, "attention partial: %s", hipGetErrorString(e));
  kap_status st = check_launch("attention partial");
  if (st != KAP_OK) return st;

  MergeArgs ma{};
  ma.row_off = c.ws.row_off;
  ma.part_o = c.ws.part_o;
  ma.part_ml = c.ws.part_ml;
  ma.out = c.out;
  ma.lse = c.lse;
  ma.out_dt = c.dtype;
  ma.q_len = c.q_len;
  ma.Hq = c.Hq;
  ma.Hkv = c.Hkv;
  ma.grp = grp;
  ma.R = R;
  dim3 mgrid(c.B * c.Hkv, R);
  const bool ph = c.dtype == KAP_BF16;  // the MFMA partials are bf16, the fp32 path's fp32
  if (c.D == 128) {
    if (ph) hipLaunchKernelGGL((attn_merge_kernel<128, true>), mgrid, dim3(256), 0, c.stream, ma);
    else hipLaunchKernelGGL((attn_merge_kernel<128, false>), mgrid, dim3(256), 0, c.stream, ma);
  } else {
    if (ph) hipLaunchKernelGGL((attn_merge_kernel<64, true>), mgrid, dim3(256), 0, c.stream, ma);
    else hipLaunchKernelGGL((attn_merge_kernel<64, false>), mgrid, dim3(256), 0, c.stream, ma);
  }
  return check_launch("attention merge");
}

}  // namespace kap
