// schedule.h -- tile scheduler of the prefill kernel (host and device).
//
// Block sparsity ("Sliding Window and Sparse Attention, from Longformer to
// CSA2", s1 last paragraph and s4 "Block-sparse attention"): attention is
// computed in tiles of bq queries x bk keys and a tile with no attended pair
// is skipped entirely; skipping a single key inside a tile saves nothing.
//
// For a query block holding positions q0 .. q1 (q1 clamped to n-1) the
// attended keys are the window band max(0, q0-w+1) .. q1 (s2 of the same page)
// and the sink positions 0 .. g-1 (s2, attention sinks).  So the visited key
// blocks are the contiguous band [kb_lo, kb_hi] plus the sink blocks
// [0, ns) that lie entirely below the band.  All of it is integer arithmetic
// evaluated in closed form by each workgroup; no block mask is stored.
#pragma once

#include <hip/hip_runtime.h>

namespace swa {

struct BandRange {
    int kb_lo;  // first key block of the window band
    int kb_hi;  // last key block of the window band (holds the diagonal)
    int ns;     // sink key blocks 0 .. ns-1 below kb_lo
    __host__ __device__ int count() const { return ns + (kb_hi - kb_lo + 1); }
    // t-th visited key block: sinks first, then the band in increasing order
    __host__ __device__ int block(int t) const { return t < ns ? t : kb_lo + (t - ns); }
};

// q0: first query position of the block, q1: last one that is < n.
__host__ __device__ inline BandRange band_range(int q0, int q1, int w, int g, int bk) {
    BandRange r;
    int lo = q0 - w + 1;
    if (lo < 0) lo = 0;
    r.kb_lo = lo / bk;
    r.kb_hi = q1 / bk;
    int ns = 0;
    if (g > 0) {
        ns = (g - 1) / bk + 1;  // blocks that hold a sink position
        if (ns > r.kb_lo) ns = r.kb_lo;  // the band already covers the rest
    }
    r.ns = ns;
    return r;
}

// A tile is FULL when every (query < n, key) pair in it is attended and none
// of its keys is a sink (so no bias is added): keys k0..k1 all at or before q0
// (causal for every row), all inside the window of the last row q1, all < n,
// and all >= g.  Everything else is an EDGE tile and is masked pair by pair.
__host__ __device__ inline bool tile_full(int q0, int q1, int k0, int k1, int n, int w, int g) {
    return k1 <= q0 && k0 >= q1 - w + 1 && k1 < n && k0 >= g;
}

// Per-pair predicate used on EDGE tiles (i = query position, j = key position).
__host__ __device__ inline bool pair_attended(int i, int j, int n, int w, int g) {
    return j <= i && j < n && (j >= i - w + 1 || j < g);
}

// Number of XCDs of an MI355X; consecutive workgroup ids are dispatched round
// robin across them, each XCD with its own L2.
constexpr int kXcds = 8;

// Workgroup id -> (unit = batch*head, query block).  Ids that land on the same
// XCD (id % 8) get a contiguous run of logical work, so neighbouring query
// blocks of one head -- which read overlapping K/V windows -- share that XCD's
// L2, and each K/V row comes from HBM about once.  Within a head the query
// blocks run from the first to the last (1-3 % faster than the reverse
// order).  Blocks start faster than one sweeps its keys, so a key's first
// reader is the block whose window begins at it: a block's first tiles miss
// in L2 and the rest of its band hits, read there by the blocks after it.  With
// grouped-query attention (group query heads per key/value head, consecutive
// units of one batch entry) the group's query heads take the same query
// block one after another, so all of them read that block's K/V tiles from
// the same L2 while they are there ("Sliding Window and Sparse Attention,
// from Longformer to CSA2", s10 glossary, GQA).  group = 1 is the order above.
__host__ __device__ inline void workgroup_order(int bid, int total, int nqb, int group, int *unit, int *qb) {
    int xcd = bid % kXcds;
    int slot = bid / kXcds;
    int per = total / kXcds;
    int rem = total % kXcds;
    int logical = (xcd < rem) ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
    const int hg = logical % group;  // query head within its group
    const int rest = logical / group;
    *qb = rest % nqb;
    *unit = (rest / nqb) * group + hg;
}

// The FULL tiles of query rows [qa, qz] (qz < n) are one contiguous run
// [*t_lo, *t_hi) of the visiting order of band r (sink blocks, which hold a
// position < g, are never FULL); an empty run is reported as [count, count).
// Closed form of the per-tile test tile_full.  klo > 0 restricts the keys
// to positions >= klo (tiles reaching below it are not FULL).
__host__ __device__ inline void full_range(const BandRange &r, int qa, int qz, int n, int w, int g, int bk,
                                           int *t_lo, int *t_hi, int klo = 0) {
    int lo_key = qz - w + 1;  // smallest key every row of the block attends in the window
    if (lo_key < g) lo_key = g;
    if (lo_key < klo) lo_key = klo;
    if (lo_key < 0) lo_key = 0;
    int kb_a = (lo_key + bk - 1) / bk;  // first block whose keys are all >= lo_key
    int kb_b = (qa + 1) / bk - 1;       // last block whose keys are all <= qa
    const int kb_n = n / bk - 1;        // last block entirely below n
    if (kb_b > kb_n) kb_b = kb_n;
    if (kb_a < r.kb_lo) kb_a = r.kb_lo;
    if (kb_b > r.kb_hi) kb_b = r.kb_hi;
    if (kb_a > kb_b) {
        *t_lo = *t_hi = r.count();
    } else {
        *t_lo = r.ns + (kb_a - r.kb_lo);
        *t_hi = r.ns + (kb_b - r.kb_lo) + 1;
    }
}

}  // namespace swa
