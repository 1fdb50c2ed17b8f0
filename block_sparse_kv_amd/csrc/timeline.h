// Per-workgroup timeline of the decode-step kernels, compiled in only with -DKVS_TIMELINE (the
// libkvs_timeline.so variant; the default library carries none of it).  Every recorded workgroup (or
// 256-lane part of one) owns a record of kTlSlots 64-bit words at
//   records + ((kind * kTlMaxWg) + index) * kTlSlots,
// index = the linear workgroup index (times the parts per workgroup, plus the part), when below
// kTlMaxWg; slot 0 holds its start, slots 1..5 the marks below and slot 6 a signature:
//   bits 0..31 index, 48..51 XCC id, 52..59 hardware CU id bits, 60..63 kind.
// Times are s_memrealtime ticks (a constant 100 MHz clock common to the device).  Marks:
//   1  the workgroup's operands have arrived (its loads waited for: the timeline build waits for
//      them at that point, which the default build need not do)
//   2  the workgroup's own work is stored (for a scoring workgroup: it has bumped the counter)
//   3  the selection made by the workgroup is stored
//   4  the chunk summary is stored (long-row scoring)
//   5  the chunk summary is made, its stores issued
// A workgroup clears its record's marks when it starts, so after several launches of a kind the
// records hold the last launch's workgroups (and those of earlier launches past its grid).
#pragma once

namespace kvs {

enum TlKind {
  kTlScoreSel = 0,   // scoring workgroups of the fused scoring + selection launch
  kTlIlStep = 1,     // Initial/Local tiles in that launch
  kTlIlWide = 2,     // Initial/Local tiles beside the wide top-k
  kTlAttn = 3,       // attention over the selected tiles
  kTlMerge = 4,      // log-sum-exp merge
  kTlWideTopk = 5,   // wide top-k selections
  kTlScore = 6,      // scoring launch of its own
  kTlTopk = 7,       // top-k launch of its own
  kTlCompact = 8,    // preselected-set compaction
  kTlMapBack = 9,    // mapping of a confined selection back to block ids
  kTlTileSel = 10,   // selections made by the selected tiles' workgroups (before their tiles)
  kTlAttnIl = 11,    // Initial/Local tiles in the selected tiles' launch
  kTlKinds = 12
};
constexpr int kTlMaxWg = 16384;
constexpr int kTlSlots = 8;

#ifdef KVS_TIMELINE
// The record of this workgroup (part of part_lanes lanes), written by the part's first lane; null in
// every other lane, past kTlMaxWg, or without a record array.
__device__ inline unsigned long long* tl_begin(unsigned long long* records, int kind, int part_lanes) {
  if (records == nullptr || (threadIdx.x % part_lanes) != 0) return nullptr;
  const unsigned long long t = __builtin_amdgcn_s_memrealtime();
  const unsigned lin = blockIdx.x + gridDim.x * (blockIdx.y + gridDim.y * blockIdx.z);
  const unsigned idx = lin * (blockDim.x / part_lanes) + threadIdx.x / part_lanes;
  if (idx >= (unsigned)kTlMaxWg) return nullptr;
  unsigned long long* r = records + ((size_t)kind * kTlMaxWg + idx) * kTlSlots;
  const unsigned xcc = __builtin_amdgcn_s_getreg(0x1814);  // hwreg(XCC_ID, 0, 4)
  const unsigned hw = __builtin_amdgcn_s_getreg(0xF804);   // hwreg(HW_ID, 0, 32)
  r[0] = t;
  r[1] = r[2] = r[3] = r[4] = r[5] = r[7] = 0ull;
  r[6] = (unsigned long long)idx | ((unsigned long long)(xcc & 15) << 48) |
         ((unsigned long long)((hw >> 8) & 0xFF) << 52) | ((unsigned long long)kind << 60);
  return r;
}
#define KVS_TL_BEGIN(P, KIND, PART) unsigned long long* kvs_tl_rec = ::kvs::tl_begin((P).tl, (KIND), (PART));
#define KVS_TL_MARK(SLOT) \
  if (kvs_tl_rec) kvs_tl_rec[SLOT] = __builtin_amdgcn_s_memrealtime();
#define KVS_TL_MARK_LOADED(SLOT) \
  {                              \
    ::kvs::wait_mem();           \
    KVS_TL_MARK(SLOT)            \
  }
#define KVS_TL_REC kvs_tl_rec
#else
#define KVS_TL_BEGIN(P, KIND, PART)
#define KVS_TL_MARK(SLOT)
#define KVS_TL_MARK_LOADED(SLOT)
#define KVS_TL_REC nullptr
#endif

}  // namespace kvs
