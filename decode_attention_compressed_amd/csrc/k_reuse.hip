// Slots for reusing rebuilt chunks across decode steps (gfx950).
//
// During generation LowRAM splits the context into chunks, picks those suited
// to the current query and reuses data it has already rebuilt (rit.work page,
// generation section).  Here a chunk's rebuilt keys U_{l,h} deq(c~) (fp16, as
// the attend kernel holds them) can be kept in a slot of a per-(sequence,
// layer, kv head) table.  Before each step, this kernel maps the step's
// selected chunks to slots:
//   - a chunk already in a slot is a hit (code slot | REUSE_HIT);
//   - the other chunks, in ascending chunk order, take the least recently used
//     slots that no hit of this step holds (older stamp first, then lower slot
//     index) and are stored there after they are rebuilt (code slot);
//   - when no such slot is left the chunk is rebuilt and not stored (code -1).
// Every used slot gets the head's new use count as its stamp.  One wave per
// (b, h), all decisions in a fixed order, so the mapping is deterministic.
#include "common.hpp"
#include "internal.hpp"

namespace lowram {

// One wave per (b, h); lanes work on selected chunks and on slots in
// parallel: hits by search, free slots ranked by (stamp, index), misses ranked
// by chunk order, miss m takes the free slot of rank m.
// grid (Hkv, B), 64 threads; dynamic LDS 4 * S + k int32.
__global__ __launch_bounds__(64) void k_reuse_assign(const int32_t *__restrict__ sel, int k,
                                                     int32_t *__restrict__ slot_chunk,
                                                     int32_t *__restrict__ slot_stamp,
                                                     int32_t *__restrict__ clock, int S, int G, int Hkv,
                                                     int layer, int32_t *__restrict__ rslot,
                                                     int32_t *__restrict__ hits_out) {
  extern __shared__ int32_t smr[];
  int32_t *ch = smr, *stp = smr + S, *used = smr + 2 * S, *by_rank = smr + 3 * S, *code = smr + 4 * S;
  const int h = blockIdx.x, b = blockIdx.y, lane = threadIdx.x;
  const long row = ((long)b * G + layer) * Hkv + h;  // table row
  const long sr = (long)b * Hkv + h;                  // selection row
  for (int i = lane; i < S; i += 64) {
    ch[i] = slot_chunk[row * S + i];
    stp[i] = slot_stamp[row * S + i];
    used[i] = 0;
  }
  const int t = clock[row] + 1;
  __syncthreads();
  // hits: each lane searches the table for its chunks (a chunk is in at most one slot)
  int hits = 0;
  for (int i = lane; i < k; i += 64) {
    const int c = sel[sr * k + i];
    int found = -1;
    for (int j = 0; j < S; ++j) found = (found < 0 && ch[j] == c) ? j : found;
    code[i] = found >= 0 ? (found | REUSE_HIT) : -1;
    if (found >= 0) used[found] = 1;
    hits += found >= 0;
  }
  __syncthreads();
  // free slots ranked by (stamp, index)
  int n_free = 0;
  for (int j = 0; j < S; ++j) n_free += used[j] == 0;
  for (int j = lane; j < S; j += 64) {
    if (used[j]) continue;
    int rank = 0;
    for (int j2 = 0; j2 < S; ++j2)
      rank += !used[j2] && (stp[j2] < stp[j] || (stp[j2] == stp[j] && j2 < j));
    by_rank[rank] = j;
  }
  __syncthreads();
  // misses in chunk order take free slots in rank order
  int before = 0;  // misses in earlier 64-chunk groups
  for (int i0 = 0; i0 < k; i0 += 64) {
    const int i = i0 + lane;
    const bool miss = i < k && code[i] == -1;
    const uint64_t mm = __ballot(miss);
    const int m = before + __popcll(mm & ((1ull << lane) - 1ull));
    if (miss && m < n_free) {
      const int v = by_rank[m];
      ch[v] = sel[sr * k + i];
      stp[v] = t;
      code[i] = v;
    }
    before += __popcll(mm);
  }
  __syncthreads();
  for (int i = lane; i < k; i += 64) {
    const int cd = code[i];
    if (cd >= 0 && (cd & REUSE_HIT)) stp[cd & ~REUSE_HIT] = t;
  }
  __syncthreads();
  for (int i = lane; i < S; i += 64) {
    slot_chunk[row * S + i] = ch[i];
    slot_stamp[row * S + i] = stp[i];
  }
  for (int i = lane; i < k; i += 64) rslot[sr * k + i] = code[i];
  for (int o = 32; o > 0; o >>= 1) hits += __shfl_xor(hits, o, 64);
  if (lane == 0) {
    clock[row] = t;
    if (hits_out) hits_out[sr] = hits;
  }
}

hipError_t launch_reuse_assign(const int32_t *sel, int k, int32_t *slot_chunk, int32_t *slot_stamp,
                               int32_t *clock, int S, int B, int G, int Hkv, int layer, int32_t *rslot,
                               int32_t *hits_out, hipStream_t st) {
  const size_t lds = sizeof(int32_t) * (4 * (size_t)S + (size_t)k);
  hipLaunchKernelGGL(k_reuse_assign, dim3(Hkv, B), dim3(64), lds, st, sel, k, slot_chunk, slot_stamp, clock, S,
                     G, Hkv, layer, rslot, hits_out);
  return hipGetLastError();
}

}  // namespace lowram
