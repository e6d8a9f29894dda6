// Work items of the chunk scan, shared by its kernels (internal header).
#pragma once

#include "common.h"
#include "kernels.h"

namespace ssd {

constexpr int kPN = kHeadDim * kDState;

// ---------------------------------------------------------------------------
// Work items
// ---------------------------------------------------------------------------
struct Item {
  int row, k, tok0, tok1, first, last, item;
  int seq0;      // first token of the item's sequence
  int64_t boff;  // batch row used for strides (0 in packed mode)
};

struct PlanView {
  const int *seq_start, *seq_end, *seq_nseg, *seq_off, *item_seq, *item_k, *n_items, *item_order;
};

__device__ __forceinline__ PlanView plan_view(const ScanPlan &plan, const char *ws) {
  const int *b = reinterpret_cast<const int *>(ws + plan.ws_plan_off);
  PlanView v;
  v.seq_start = b;
  v.seq_end = b + plan.rows;
  v.seq_nseg = b + 2 * plan.rows;
  v.seq_off = b + 3 * plan.rows;
  v.item_seq = b + 4 * plan.rows;
  v.item_k = v.item_seq + plan.items;
  v.n_items = v.item_k + plan.items;
  v.item_order = v.n_items + 1;
  return v;
}

__device__ __forceinline__ bool get_item(const ScanParams &p, const ScanPlan &plan,
                                         const char *ws, int item, Item &it) {
  it.item = item;
  if (!plan.packed) {
    it.row = item / plan.nseg;
    it.k = item % plan.nseg;
    it.tok0 = it.k * plan.seg_len;
    it.tok1 = min(p.L, it.tok0 + plan.seg_len);
    it.first = it.k == 0;
    it.last = it.k == plan.nseg - 1;
    it.boff = it.row;
    it.seq0 = 0;
    return true;
  }
  const PlanView v = plan_view(plan, ws);
  if (item >= *v.n_items) return false;
  it.row = v.item_seq[item];
  it.k = v.item_k[item];
  const int start = v.seq_start[it.row], end = v.seq_end[it.row];
  it.tok0 = start + it.k * plan.seg_len;
  it.tok1 = min(end, it.tok0 + plan.seg_len);
  it.first = it.k == 0;
  it.last = it.k == v.seq_nseg[it.row] - 1;
  it.boff = 0;
  it.seq0 = start;
  return true;
}

// blockIdx -> (item, head).  Workgroups go to the XCDs round-robin by
// blockIdx, and each XCD starts its workgroups in blockIdx order.
//  * Batch mode (items of equal length): XCD x gets a contiguous range of the
//    work list, ordered item-major, then group, then head.
//  * Packed mode (items of any length): the (item, group) units, longest item
//    first, are dealt round-robin over the XCDs, and each XCD runs its units'
//    heads one unit after the other.  The long items start first and every
//    XCD gets a share of each length, so the last workgroups to finish are
//    short ones; a unit's heads (which read the same B and C) stay on one XCD.
__device__ __forceinline__ bool map_workgroup(const ScanParams &p, const ScanPlan &plan, const char *ws,
                                              int &item, int &h, int &g) {
  const int hpg = p.H / p.G;
  if (plan.packed) {
    const int pos = blockIdx.x / kNumXCD;
    const int k = (pos / hpg) * kNumXCD + blockIdx.x % kNumXCD;  // unit rank
    const int rank = k / p.G;
    const PlanView v = plan_view(plan, ws);
    if (rank >= *v.n_items) return false;
    item = v.item_order[rank];
    g = k % p.G;
    h = g * hpg + pos % hpg;
    return true;
  }
  const int total = plan.items * p.H;
  const int per_xcd = gridDim.x / kNumXCD;
  const int w = (blockIdx.x % kNumXCD) * per_xcd + blockIdx.x / kNumXCD;
  if (w >= total) return false;
  const int hl = w % hpg;
  const int t = w / hpg;
  g = t % p.G;
  item = t / p.G;
  h = g * hpg + hl;
  return true;
}

// Workgroups a scan launch needs for this plan (a multiple of the XCD count).
inline unsigned scan_grid_size(const ScanParams &p, const ScanPlan &plan) {
  const long long x = kNumXCD;
  if (plan.packed) {
    const long long units = (long long)plan.items * p.G;
    return (unsigned)((units + x - 1) / x * x * (p.H / p.G));
  }
  const long long total = (long long)plan.items * p.H;
  return (unsigned)((total + x - 1) / x * x);
}

__device__ __forceinline__ float *ws_f32(const ScanPlan &plan, char *ws, size_t off) {
  return reinterpret_cast<float *>(ws + off);
}


hipError_t launch_chunk_scan_bf16(const ScanParams &p, const ScanPlan &plan, char *ws, unsigned nblk, bool full,
                                  hipStream_t stream);

}  // namespace ssd
