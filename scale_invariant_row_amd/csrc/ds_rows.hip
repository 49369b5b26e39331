// The C ABI of include/ds_rows.h: argument checks, kernel shape and grid
// choice, and the staging of ragged weight descriptors.
//
// Every check runs before the first HIP call, so a refused call has touched
// neither the device nor the stream.
#include "ds_rows.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "launch.hpp"
#include "row_kernels.hpp"

namespace dsr {

// ------------------------------------------------ scalar-gain totals
//
// A scalar gain's gradient is the sum of its rows' shares (written by
// rownorm_backward_kernel).  One workgroup of 256 threads per matrix: thread
// k adds rows k, k + 256, ... in order, then the 256 partial sums are
// combined by the wave tree and the four wave totals in order.  The order
// depends on the row count alone.

struct TotalTask {
  const float* shares;
  float* total;
  int64_t rows;
};
constexpr int kTotalTasks = 64;
struct TotalArgs {
  int32_t ntasks;
  TotalTask tasks[kTotalTasks];
};
static_assert(sizeof(TotalArgs) <= 4096, "kernel arguments are limited to 4 KiB");

__global__ void __launch_bounds__(256) row_total_kernel(const TotalArgs args) {
  __shared__ float part[4];
  const TotalTask t = args.tasks[blockIdx.x];
  float a = 0.f;
  for (int64_t i = threadIdx.x; i < t.rows; i += 256) a += t.shares[i];
  a = wave_sum(a);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) part[wave] = a;
  __syncthreads();
  if (threadIdx.x == 0) *t.total = ((part[0] + part[1]) + part[2]) + part[3];
}

}  // namespace dsr

namespace {

using dsr::Shape;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// [a, a + na) and [b, b + nb) share a byte.
bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return na > 0 && nb > 0 && x < y + nb && y < x + na;
}

// Output buffer may be exactly the input buffer, or disjoint from it.
bool same_or_disjoint(const void* out, const void* in, size_t n) {
  return in == nullptr || out == in || !overlaps(out, n, in, n);
}

bool finite_nonneg(float v) { return std::isfinite(v) && v >= 0.f; }

// rows x cols elements of `esize` bytes; cols a multiple of `mult`.
int check_matrix(int64_t rows, int64_t cols, int64_t mult, int64_t esize) {
  if (rows < 0 || cols < mult || cols > DS_MAX_COLS || cols % mult != 0) return DS_ERR_SHAPE;
  if (rows > (INT64_MAX / 8) / (cols * esize)) return DS_ERR_SHAPE;
  return DS_OK;
}

// Compute units of the current device, cached per device.
int device_cus(int* cus) {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DS_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it == cache.end()) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      return DS_ERR_DEVICE;
    it = cache.emplace(dev, n).first;
  }
  *cus = it->second;
  return DS_OK;
}

// Workgroups for `units` row groups (or items): one each, up to 64 per
// compute unit in a launch, well above what the chip holds at once.  Past
// that the ragged kernels loop (grid-stride) and the row kernels run as
// several launches (launch_in_pieces).  A cap of 2^20 workgroups measured
// the same (GPT-2's 768-wide linears, 18,432 items: 89.6-89.9 against
// 89.8-90.3 us forward).  DS_ROWS_TEST_MAX_GROUPS lowers the cap: a test
// hook that runs the several-launch and grid-stride paths at small sizes.
int64_t max_launch_groups(int cus) {
  const int64_t cap = (int64_t)cus * 64;
  const char* e = std::getenv("DS_ROWS_TEST_MAX_GROUPS");
  if (e != nullptr) {
    const long long v = std::atoll(e);
    if (v >= 1 && v < cap) return v;
  }
  return cap;
}

int grid_for(int64_t units, int cus) {
  return (int)std::max<int64_t>(1, std::min(units, max_launch_groups(cus)));
}

int launch_status(hipError_t e) { return e == hipSuccess ? DS_OK : DS_ERR_LAUNCH; }

// For kernels that take one row group per workgroup, with no grid-stride
// loop: launch(r0, n) over rows [r0, r0 + n), in pieces of at most the grid
// cap of row groups (rows_per_group rows each).
template <class F>
hipError_t launch_in_pieces(int64_t rows, int rows_per_group, int cus, F&& launch) {
  const int64_t piece = max_launch_groups(cus) * rows_per_group;
  for (int64_t r0 = 0; r0 < rows; r0 += piece) {
    const hipError_t e = launch(r0, std::min<int64_t>(piece, rows - r0));
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// ----------------------------------------------------- descriptor staging
//
// A ring of pinned host + device buffers per device.  A slot is filled on the
// host, copied to the device on the caller's stream, read by the kernels, and
// handed out again only after an event recorded behind those kernels has
// completed; a slot whose copy or launch failed is returned at once.

constexpr int kSlots = 8;

struct Slot {
  void* host = nullptr;
  void* dev = nullptr;
  size_t cap = 0;
  hipEvent_t ev = nullptr;
  bool busy = false;      // handed out, not yet returned
  bool pending = false;   // returned with work in flight behind `ev`
};

struct Ring {
  std::mutex mu;
  Slot slot[kSlots];
  int next = 0;
};

Ring* ring_for_current_device() {
  static std::mutex mu;
  static std::map<int, Ring*> rings;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  Ring*& r = rings[dev];
  if (r == nullptr) r = new Ring();   // lives until the process ends
  return r;
}

// Failure injection for the tests of the staging path.  DS_ROWS_TEST_FAIL
// names one step to fail as if the runtime had refused it: "alloc" (the
// slot's buffers), "copy" (the table's upload) or "launch" (the first
// kernel launch after the upload).  Read only when a call stages a table.
enum class Fail { kNone, kAlloc, kCopy, kLaunch };

Fail injected_failure() {
  const char* f = std::getenv("DS_ROWS_TEST_FAIL");
  if (f == nullptr) return Fail::kNone;
  if (std::strcmp(f, "alloc") == 0) return Fail::kAlloc;
  if (std::strcmp(f, "copy") == 0) return Fail::kCopy;
  if (std::strcmp(f, "launch") == 0) return Fail::kLaunch;
  return Fail::kNone;
}

int grow(Slot& s, size_t bytes, Fail fail) {
  if (fail == Fail::kAlloc) return DS_ERR_ALLOC;
  if (s.ev == nullptr && hipEventCreateWithFlags(&s.ev, hipEventDisableTiming) != hipSuccess) {
    s.ev = nullptr;
    return DS_ERR_ALLOC;
  }
  if (s.cap >= bytes) return DS_OK;
  size_t cap = std::max<size_t>(bytes, 4096);
  void* h = nullptr;
  void* d = nullptr;
  if (hipHostMalloc(&h, cap, hipHostMallocDefault) != hipSuccess) return DS_ERR_ALLOC;
  if (hipMalloc(&d, cap) != hipSuccess) {
    (void)hipHostFree(h);
    return DS_ERR_ALLOC;
  }
  if (s.host) (void)hipHostFree(s.host);
  if (s.dev) (void)hipFree(s.dev);
  s.host = h;
  s.dev = d;
  s.cap = cap;
  return DS_OK;
}

int acquire(Ring& r, size_t bytes, int* out, Fail fail) {
  std::lock_guard<std::mutex> lock(r.mu);
  int pick = -1;
  for (int t = 0; t < kSlots && pick < 0; ++t) {
    int i = (r.next + t) % kSlots;
    Slot& s = r.slot[i];
    if (s.busy) continue;
    if (s.pending) {
      if (hipEventQuery(s.ev) != hipSuccess) continue;   // still in flight
      s.pending = false;
    }
    pick = i;
  }
  if (pick < 0) {                 // every slot in flight: wait for the oldest one
    for (int t = 0; t < kSlots && pick < 0; ++t) {
      int i = (r.next + t) % kSlots;
      if (!r.slot[i].busy) pick = i;
    }
    if (pick < 0) return DS_ERR_ALLOC;
    if (hipEventSynchronize(r.slot[pick].ev) != hipSuccess) return DS_ERR_LAUNCH;
    r.slot[pick].pending = false;
  }
  int st = grow(r.slot[pick], bytes, fail);
  if (st != DS_OK) return st;
  r.slot[pick].busy = true;
  r.next = (pick + 1) % kSlots;
  *out = pick;
  return DS_OK;
}

// Return a slot: with `enqueued` work behind an event on `stream`, else at once.
void release(Ring& r, int i, bool enqueued, hipStream_t stream) {
  std::lock_guard<std::mutex> lock(r.mu);
  Slot& s = r.slot[i];
  if (enqueued) {
    if (hipEventRecord(s.ev, stream) == hipSuccess) {
      s.pending = true;
    } else {
      (void)hipStreamSynchronize(stream);   // no event: wait the work out here
      s.pending = false;
    }
  }
  s.busy = false;
}


// ------------------------------------------------------ ragged weight calls

// Byte ranges [first, second) that a call reads and writes.
using Range = std::pair<uintptr_t, uintptr_t>;

void add_range(std::vector<Range>& v, const void* p, size_t bytes) {
  if (p == nullptr || bytes == 0) return;
  auto a = reinterpret_cast<uintptr_t>(p);
  v.emplace_back(a, a + bytes);
}

// No two output ranges share a byte, and no output shares a byte with any
// input (of its own matrix or another's): every matrix of a ragged call runs
// concurrently with the others.
bool outputs_disjoint(std::vector<Range>& outs, std::vector<Range>& ins) {
  std::sort(outs.begin(), outs.end());
  for (size_t i = 1; i < outs.size(); ++i)
    if (outs[i].first < outs[i - 1].second) return false;
  std::sort(ins.begin(), ins.end());
  size_t j = 0;
  uintptr_t reach = 0;          // furthest end among inputs starting before the current output
  for (const Range& o : outs) {
    while (j < ins.size() && ins[j].first < o.second) reach = std::max(reach, ins[j++].second);
    if (reach > o.first) return false;
  }
  return true;
}

template <class Task>
using RaggedLauncher = hipError_t (*)(Shape, const dsr::TaskArgs<Task>&, int, hipStream_t);

// The launches over the matrices' tasks.  Matrices of one kernel shape form
// a class.  Small classes of contiguous rows that share a workgroup size (up
// to kMaxMixedThreads) run in one mixed-shape launch, each task carrying its
// shape key; every other class (a large one, 1,024-thread rows, a
// column-block tile width) runs in its shape's own kernel.  A launch of at
// most kInlineTasks matrices carries its table inside the kernel arguments;
// larger launches share one table (tasks, then their first items as a
// compact int32 array) staged through the ring and copied on the stream
// first.
//
// With `inline_only` every launch carries its table in the kernel arguments:
// a group of more than kInlineTasks matrices is split into launches of at
// most that many, so the call touches no library memory (the ring is never
// used).  A matrix's bits do not depend on the launch it lands in.  A call
// that would stage a table on a stream being captured into a graph is
// planned this way instead.
template <class Task>
int launch_ragged(const std::vector<std::pair<Shape, Task>>& mats, RaggedLauncher<Task> launch,
                  hipStream_t hs, bool inline_only = false) {
  if (mats.empty()) return DS_OK;
  std::map<int, std::vector<size_t>> classes;     // shape key -> indices into mats
  std::map<int, int64_t> class_items;
  for (size_t i = 0; i < mats.size(); ++i) {
    const Shape& s = mats[i].first;
    classes[s.key()].push_back(i);
    int64_t& n = class_items[s.key()];
    n += (mats[i].second.rows + s.rows_per_block() - 1) / s.rows_per_block();
    if (n > INT32_MAX) return DS_ERR_SHAPE;
  }
  int cus = 0;
  int st = device_cus(&cus);
  if (st != DS_OK) return st;
  // launch group (-workgroup size for a mixed launch, else the shape key)
  // -> shape key -> indices into mats
  std::map<int, std::map<int, std::vector<size_t>>> groups;
  for (auto& kv : classes) {
    const Shape& s = mats[kv.second.front()].first;
    const bool small = class_items[kv.first] < (int64_t)dsr::kMixedItemsPerCu * cus;
    const bool mixable = s.units == 0 && s.threads() <= dsr::kMaxMixedThreads && small;
    groups[mixable ? -s.threads() : kv.first][kv.first] = kv.second;
  }

  std::vector<Task> table;
  struct Launch { Shape s; size_t first; int ntasks; int nitems; };
  std::vector<Launch> launches;
  for (auto& grp : groups) {
    Shape ls = mats[grp.second.begin()->second.front()].first;
    if (grp.second.size() > 1) ls.mixed = ls.threads();
    std::vector<size_t> order;
    for (auto& cls : grp.second) order.insert(order.end(), cls.second.begin(), cls.second.end());
    // Column blocks: tallest matrices first.  Workgroups start in item order
    // and a tile's time grows with its stored rows, so the tall tiles (GPT-2's
    // 3,072-row MLP projections) start early instead of running alone at the
    // end: 146 instead of 172 us forward on GPT-2's Conv1D set.  (Row items
    // are short; their call order measured as fast.)  The order of the tasks
    // changes no result.
    if (ls.units > 0)
      std::stable_sort(order.begin(), order.end(), [&](size_t x, size_t y) {
        return mats[x].second.cols / mats[x].second.seg > mats[y].second.cols / mats[y].second.seg;
      });
    const size_t per_launch = inline_only ? (size_t)dsr::kInlineTasks : order.size();
    for (size_t first = 0; first < order.size(); first += per_launch) {
      Launch L{ls, table.size(), 0, 0};
      int64_t items = 0;
      for (size_t k = first; k < std::min(order.size(), first + per_launch); ++k) {
        const size_t i = order[k];
        const int R = mats[i].first.rows_per_block();
        Task t = mats[i].second;
        t.item_begin = (int32_t)items;
        t.shape = mats[i].first.key();
        items += (t.rows + R - 1) / R;
        if (items > INT32_MAX) return DS_ERR_SHAPE;
        table.push_back(t);
        ++L.ntasks;
      }
      L.nitems = (int)items;
      launches.push_back(L);
    }
  }

  size_t staged_tasks = 0;
  for (const Launch& L : launches)
    if (L.ntasks > dsr::kInlineTasks) staged_tasks += (size_t)L.ntasks;

  if (staged_tasks > 0) {
    // A staged table is copied from a reusable host slot: a graph replay
    // would copy whatever that slot holds by then.  On a capturing stream
    // the call is planned again with every table in the kernel arguments
    // (more launches, the same bits); nothing has been enqueued yet.
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(hs, &cap) != hipSuccess) return DS_ERR_LAUNCH;
    if (cap != hipStreamCaptureStatusNone) return launch_ragged(mats, launch, hs, true);
  }
  Ring* ring = nullptr;
  int slot = -1;
  const Task* dev_tasks = nullptr;
  const int32_t* dev_begins = nullptr;
  const Fail fail = staged_tasks > 0 ? injected_failure() : Fail::kNone;
  (void)hipGetLastError();
  if (staged_tasks > 0) {
    ring = ring_for_current_device();
    if (ring == nullptr) return DS_ERR_DEVICE;
    const size_t task_bytes = staged_tasks * sizeof(Task);
    const size_t bytes = task_bytes + staged_tasks * sizeof(int32_t);
    if ((st = acquire(*ring, bytes, &slot, fail)) != DS_OK) return st;
    Slot& sl = ring->slot[slot];
    auto* host_tasks = static_cast<Task*>(sl.host);
    auto* host_begins = reinterpret_cast<int32_t*>(static_cast<char*>(sl.host) + task_bytes);
    size_t k = 0;
    for (const Launch& L : launches) {
      if (L.ntasks <= dsr::kInlineTasks) continue;
      for (int i = 0; i < L.ntasks; ++i, ++k) {
        host_tasks[k] = table[L.first + i];
        host_begins[k] = table[L.first + i].item_begin;
      }
    }
    if (fail == Fail::kCopy ||
        hipMemcpyAsync(sl.dev, sl.host, bytes, hipMemcpyHostToDevice, hs) != hipSuccess) {
      release(*ring, slot, false, hs);        // nothing enqueued: refund the slot
      return DS_ERR_LAUNCH;
    }
    dev_tasks = static_cast<const Task*>(sl.dev);
    dev_begins = reinterpret_cast<const int32_t*>(static_cast<const char*>(sl.dev) + task_bytes);
  }

  int result = DS_OK;
  size_t staged_at = 0;
  for (const Launch& L : launches) {
    dsr::TaskArgs<Task> args{};
    args.ntasks = L.ntasks;
    args.nitems = L.nitems;
    if (L.ntasks <= dsr::kInlineTasks) {
      args.tasks = nullptr;
      args.begins = nullptr;
      for (int i = 0; i < L.ntasks; ++i) {
        args.inline_tasks[i] = table[L.first + i];
        args.inline_begins[i] = table[L.first + i].item_begin;
      }
    } else {
      args.tasks = dev_tasks + staged_at;
      args.begins = dev_begins + staged_at;
      staged_at += (size_t)L.ntasks;
    }
    if (fail == Fail::kLaunch || launch(L.s, args, grid_for(L.nitems, cus), hs) != hipSuccess) {
      result = DS_ERR_LAUNCH;
      break;
    }
  }
  if (ring != nullptr) release(*ring, slot, true, hs);   // the copy is in flight either way
  return result;
}

// The weight launchers: row kernels, or a column-block kernel (single-pass
// or two-pass) for a column-block shape class.
hipError_t launch_rownorm_any(Shape s, const dsr::TaskArgs<dsr::RownormTask>& a, int grid,
                              hipStream_t hs) {
  if (s.col1 > 0) return dsr::launch_colblock1_rownorm(a, grid, hs);
  return s.units > 0 ? dsr::launch_colblock_rownorm(a, grid, hs) : dsr::launch_rownorm(s, a, grid, hs);
}

hipError_t launch_rownorm_backward_any(Shape s, const dsr::TaskArgs<dsr::RownormGradTask>& a,
                                       int grid, hipStream_t hs) {
  if (s.col1 > 0) return dsr::launch_colblock1_rownorm_backward(a, grid, hs);
  return s.units > 0 ? dsr::launch_colblock_rownorm_backward(a, grid, hs)
                     : dsr::launch_rownorm_backward(s, a, grid, hs);
}

hipError_t launch_project_any(Shape s, const dsr::TaskArgs<dsr::RescaleTask>& a, int grid,
                              hipStream_t hs) {
  if (s.col1 > 0) return dsr::launch_colblock1_rescale(false, a, grid, hs);
  return s.units > 0 ? dsr::launch_colblock_rescale(false, a, grid, hs)
                     : dsr::launch_rescale_project(s, a, grid, hs);
}

hipError_t launch_after_step_any(Shape s, const dsr::TaskArgs<dsr::RescaleTask>& a, int grid,
                                 hipStream_t hs) {
  if (s.col1 > 0) return dsr::launch_colblock1_rescale(true, a, grid, hs);
  return s.units > 0 ? dsr::launch_colblock_rescale(true, a, grid, hs)
                     : dsr::launch_rescale_after_step(s, a, grid, hs);
}

// An fp32 weight matrix: rows >= 0 and 1 <= cols <= DS_MAX_COLS; a width that
// is not a multiple of 4 takes the single-element path, up to kMaxElemCols.
// Returns the kernel shape in *s, and the alignment its fp32 and bf16
// buffers need (16 bytes on the vector path; 4 and 2 on the element path).
int check_weight(int64_t rows, int64_t cols, Shape* s, uintptr_t* a32, uintptr_t* a16) {
  int st = check_matrix(rows, cols, 1, 4);
  if (st != DS_OK) return st;
  *s = dsr::pick_weight_shape(cols);
  if (!s->ok()) return DS_ERR_SHAPE;
  *a32 = s->NE == 4 ? 16 : 4;
  *a16 = s->NE == 4 ? 16 : 2;
  return DS_OK;
}

// A weight's layout: contiguous rows (seg == 0; check_weight), or a column
// block: `rows` units of cols = A * seg values, unit u owning the seg values
// at u * seg of each of the A stored rows, ld elements apart.  Returns the
// shape, the alignments (4-byte fp32, 2-byte bf16 for column blocks) and the
// span, in elements, from the first value to one past the last.
int check_layout(int64_t rows, int64_t cols, int32_t seg, int64_t ld, Shape* s,
                 uintptr_t* a32, uintptr_t* a16, int64_t* span) {
  if (seg == 0) {
    int st = check_weight(rows, cols, s, a32, a16);
    *span = rows * cols;
    return st;
  }
  int st = check_matrix(rows, cols, 1, 4);
  if (st != DS_OK) return st;
  if (seg < 0 || seg > dsr::kMaxSeg || cols % seg != 0) return DS_ERR_SHAPE;
  const int64_t A = cols / seg;
  if (ld < rows * seg || (A > 1 && ld > (INT64_MAX / 8) / (A - 1))) return DS_ERR_SHAPE;
  *span = (A - 1) * ld + rows * seg;
  *s = dsr::colblock_shape(seg);
  *a32 = 4;
  *a16 = 2;
  return DS_OK;
}

// A column block that the seg-1 kernel takes: seg 1, a unit count and ld
// that are multiples of 4, and 16-byte-aligned fp32 buffers (8 for bf16; the
// caller checks them into `vec_aligned`).  Its tiles are single-pass (4 lanes
// units) when col1_single admits the matrix, else two-pass (64 units).
// Others keep the two-pass kernel's shape `s`.
Shape single_pass(Shape s, int K, int lanes, int64_t rows, int64_t cols, int32_t seg, int64_t ld,
                  bool vec_aligned) {
  if (s.units == 0 || seg != 1 || rows % 4 != 0 || ld % 4 != 0 || !vec_aligned) return s;
  Shape c{};
  c.units = dsr::col1_single(cols, ld, K, lanes) ? 4 * lanes : 64;
  c.col1 = K * 100 + lanes;
  return c;
}

bool gain_mode_ok(int32_t m) {
  return m == DS_GAIN_ROW || m == DS_GAIN_SCALAR || m == DS_GAIN_NONE;
}

size_t gain_bytes(int32_t mode, int64_t rows) {
  return mode == DS_GAIN_ROW ? (size_t)rows * 4 : mode == DS_GAIN_SCALAR ? 4 : 0;
}

// The l2_rows gradient's buffers: dx may be exactly x, r or dy (each row is
// held in registers before its store), or disjoint from all three.
int check_l2_backward(const uint16_t* x, const uint16_t* r, const uint16_t* dy, uint16_t* dx,
                      int64_t rows, int64_t cols, float eps) {
  int st = check_matrix(rows, cols, 8, 2);
  if (st != DS_OK) return st;
  if (!finite_nonneg(eps)) return DS_ERR_ARG;
  if (rows == 0) return DS_OK;
  if (x == nullptr || dy == nullptr || dx == nullptr) return DS_ERR_NULL;
  if (!aligned(x, 16) || !aligned(dy, 16) || !aligned(dx, 16) || (r != nullptr && !aligned(r, 16)))
    return DS_ERR_ALIGN;
  const size_t bytes = (size_t)rows * (size_t)cols * 2;
  if (!same_or_disjoint(dx, x, bytes) || !same_or_disjoint(dx, r, bytes) ||
      !same_or_disjoint(dx, dy, bytes))
    return DS_ERR_ARG;
  return DS_OK;
}

}  // namespace

extern "C" {

int ds_version(void) { return DS_ROWS_VERSION; }

const char* ds_status_string(int status) {
  switch (status) {
    case DS_OK: return "DS_OK: success";
    case DS_ERR_NULL: return "DS_ERR_NULL: a required pointer is NULL";
    case DS_ERR_SHAPE: return "DS_ERR_SHAPE: rows/cols out of range or cols not a multiple of the vector width";
    case DS_ERR_ALIGN: return "DS_ERR_ALIGN: a pointer is misaligned";
    case DS_ERR_ARG: return "DS_ERR_ARG: invalid eps/radius/count, or partly overlapping buffers";
    case DS_ERR_ALLOC: return "DS_ERR_ALLOC: could not allocate the descriptor staging buffer";
    case DS_ERR_LAUNCH: return "DS_ERR_LAUNCH: the HIP runtime reported an error";
    case DS_ERR_DEVICE: return "DS_ERR_DEVICE: no usable HIP device";
    case DS_ERR_CAPTURE: return "DS_ERR_CAPTURE: reserved (a ragged call on a capturing stream now splits its launches instead)";
    case DS_ERR_SCRATCH: return "DS_ERR_SCRATCH: the call needs more library scratch than DS_SCRATCH_FLOATS (1,048,576 scalar-gain rows)";
    default: return "unknown ds_rows status";
  }
}

namespace {

using ForwardLaunch = hipError_t (*)(Shape, const void*, const void*, void*, int64_t, int, float,
                                     int, hipStream_t);

// l2_rows and rms_rows: the same checks, shape and grid.
int norm_rows(ForwardLaunch launch, const uint16_t* x, const uint16_t* r, uint16_t* y,
              int64_t rows, int64_t cols, float eps, ds_stream_t stream) {
  int st = check_matrix(rows, cols, 8, 2);
  if (st != DS_OK) return st;
  if (!finite_nonneg(eps)) return DS_ERR_ARG;
  if (rows == 0) return DS_OK;
  if (x == nullptr || y == nullptr) return DS_ERR_NULL;
  if (!aligned(x, 16) || !aligned(y, 16) || (r != nullptr && !aligned(r, 16))) return DS_ERR_ALIGN;
  const size_t bytes = (size_t)rows * (size_t)cols * 2;
  if (!same_or_disjoint(y, x, bytes) || !same_or_disjoint(y, r, bytes)) return DS_ERR_ARG;

  const Shape s = dsr::pick_bf16_shape(cols / 8);
  if (!s.ok()) return DS_ERR_SHAPE;
  int cus = 0;
  if ((st = device_cus(&cus)) != DS_OK) return st;
  const int rpg = s.rows_per_block();
  (void)hipGetLastError();   // start from a clean error state
  return launch_status(launch_in_pieces(rows, rpg, cus, [&](int64_t r0, int64_t n) {
    const int64_t at = r0 * cols;
    return launch(s, x + at, r != nullptr ? r + at : nullptr, y + at, n, (int)(cols / 8), eps,
                  (int)((n + rpg - 1) / rpg), (hipStream_t)stream);
  }));
}

using BackwardLaunch = hipError_t (*)(Shape, const void*, const void*, const void*, void*,
                                      int64_t, int, float, int, hipStream_t);

int norm_rows_backward(BackwardLaunch launch, const uint16_t* x, const uint16_t* r,
                       const uint16_t* dy, uint16_t* dx, int64_t rows, int64_t cols, float eps,
                       ds_stream_t stream) {
  int st = check_l2_backward(x, r, dy, dx, rows, cols, eps);
  if (st != DS_OK || rows == 0) return st;
  const Shape s = dsr::pick_bf16_shape(cols / 8);
  if (!s.ok()) return DS_ERR_SHAPE;
  int cus = 0;
  if ((st = device_cus(&cus)) != DS_OK) return st;
  const int rpg = s.rows_per_block();
  (void)hipGetLastError();
  return launch_status(launch_in_pieces(rows, rpg, cus, [&](int64_t r0, int64_t n) {
    const int64_t at = r0 * cols;
    return launch(s, x + at, r != nullptr ? r + at : nullptr, dy + at, dx + at, n,
                  (int)(cols / 8), eps, (int)((n + rpg - 1) / rpg), (hipStream_t)stream);
  }));
}

}  // namespace

int ds_l2_rows(const uint16_t* x, const uint16_t* r, uint16_t* y, int64_t rows, int64_t cols,
               float eps, ds_stream_t stream) {
  return norm_rows(dsr::launch_l2_rows, x, r, y, rows, cols, eps, stream);
}

int ds_rms_rows(const uint16_t* x, const uint16_t* r, uint16_t* y, int64_t rows, int64_t cols,
                float eps, ds_stream_t stream) {
  return norm_rows(dsr::launch_rms_rows, x, r, y, rows, cols, eps, stream);
}

int ds_slerp_rows(const uint16_t* res, const uint16_t* out, const float* alpha, uint16_t* h,
                  int64_t rows, int64_t cols, float eps, ds_stream_t stream) {
  int st = check_matrix(rows, cols, 8, 2);
  if (st != DS_OK) return st;
  if (!finite_nonneg(eps)) return DS_ERR_ARG;
  if (rows == 0) return DS_OK;
  if (res == nullptr || out == nullptr || alpha == nullptr || h == nullptr) return DS_ERR_NULL;
  if (!aligned(res, 16) || !aligned(out, 16) || !aligned(alpha, 16) || !aligned(h, 16))
    return DS_ERR_ALIGN;
  const size_t bytes = (size_t)rows * (size_t)cols * 2;
  if (!same_or_disjoint(h, res, bytes) || !same_or_disjoint(h, out, bytes)) return DS_ERR_ARG;
  if (overlaps(h, bytes, alpha, (size_t)cols * 4)) return DS_ERR_ARG;

  const Shape s = dsr::pick_bf16_shape(cols / 8);
  if (!s.ok()) return DS_ERR_SHAPE;
  int cus = 0;
  if ((st = device_cus(&cus)) != DS_OK) return st;
  const int rpg = s.rows_per_block();
  (void)hipGetLastError();
  return launch_status(launch_in_pieces(rows, rpg, cus, [&](int64_t r0, int64_t n) {
    const int64_t at = r0 * cols;
    return dsr::launch_slerp_rows(s, res + at, out + at, alpha, h + at, n, (int)(cols / 8), eps,
                                  (int)((n + rpg - 1) / rpg), (hipStream_t)stream);
  }));
}

namespace {

// Checks shared by the two activation rows: two bf16 input rows, one or two
// fp32 column vectors, one bf16 output that may be exactly either input.
int check_act(const uint16_t* a, const uint16_t* b, const float* s0, const float* s1, uint16_t* y,
              int64_t rows, int64_t cols, float eps, bool two_scales) {
  int st = check_matrix(rows, cols, 8, 2);
  if (st != DS_OK) return st;
  if (!finite_nonneg(eps)) return DS_ERR_ARG;
  if (rows == 0) return DS_OK;
  if (a == nullptr || b == nullptr || s0 == nullptr || y == nullptr || (two_scales && s1 == nullptr))
    return DS_ERR_NULL;
  if (!aligned(a, 16) || !aligned(b, 16) || !aligned(s0, 16) || !aligned(y, 16) ||
      (two_scales && !aligned(s1, 16)))
    return DS_ERR_ALIGN;
  const size_t bytes = (size_t)rows * (size_t)cols * 2;
  if (!same_or_disjoint(y, a, bytes) || !same_or_disjoint(y, b, bytes)) return DS_ERR_ARG;
  if (overlaps(y, bytes, s0, (size_t)cols * 4) || (two_scales && overlaps(y, bytes, s1, (size_t)cols * 4)))
    return DS_ERR_ARG;
  return DS_OK;
}

}  // namespace

int ds_gate_l2_rows(const uint16_t* o, const uint16_t* g, const float* sg, uint16_t* y,
                    int64_t rows, int64_t cols, float eps, ds_stream_t stream) {
  int st = check_act(o, g, sg, nullptr, y, rows, cols, eps, false);
  if (st != DS_OK || rows == 0) return st;
  const Shape s = dsr::pick_act_shape(cols / 8);
  if (!s.ok()) return DS_ERR_SHAPE;
  int cus = 0;
  if ((st = device_cus(&cus)) != DS_OK) return st;
  const int rpg = s.rows_per_block();
  (void)hipGetLastError();
  return launch_status(launch_in_pieces(rows, rpg, cus, [&](int64_t r0, int64_t n) {
    const int64_t at = r0 * cols;
    return dsr::launch_gate_l2_rows(s, o + at, g + at, sg, y + at, n, (int)(cols / 8), eps,
                                    (int)((n + rpg - 1) / rpg), (hipStream_t)stream);
  }));
}

int ds_swiglu_l2_rows(const uint16_t* g, const uint16_t* u, const float* sug, const float* suu,
                      uint16_t* y, int64_t rows, int64_t cols, float eps, ds_stream_t stream) {
  int st = check_act(g, u, sug, suu, y, rows, cols, eps, true);
  if (st != DS_OK || rows == 0) return st;
  const Shape s = dsr::pick_act_shape(cols / 8);
  if (!s.ok()) return DS_ERR_SHAPE;
  int cus = 0;
  if ((st = device_cus(&cus)) != DS_OK) return st;
  const int rpg = s.rows_per_block();
  (void)hipGetLastError();
  return launch_status(launch_in_pieces(rows, rpg, cus, [&](int64_t r0, int64_t n) {
    const int64_t at = r0 * cols;
    return dsr::launch_swiglu_l2_rows(s, g + at, u + at, sug, suu, y + at, n, (int)(cols / 8),
                                      eps, (int)((n + rpg - 1) / rpg), cus,
                                      (hipStream_t)stream);
  }));
}

namespace {

// Bytes a strided [rows, width] bf16 view spans.
size_t span_bytes(int64_t rows, int64_t ld, int64_t width) {
  return rows == 0 ? 0 : ((size_t)(rows - 1) * (size_t)ld + (size_t)width) * 2;
}

int64_t floor_div(int64_t a, int64_t b) { return a / b - ((a % b != 0) && ((a < 0) != (b < 0))); }

// Two [rows, wa] and [rows, wb] bf16 views at a and b share an element.  With
// one row stride ld (>= wa, wb) the test is exact: element (ra, ca) of a is
// element (rb, cb) of b when (ra - rb) ld = de + cb - ca, de = (b - a) / 2,
// so some multiple k ld with |k| < rows must lie in (de - wa, de + wb).
// Otherwise it compares the spans.
bool views_overlap(const void* a, int64_t lda, int64_t wa, const void* b, int64_t ldb, int64_t wb,
                   int64_t rows) {
  if (rows == 0 || wa == 0 || wb == 0 || a == nullptr || b == nullptr) return false;
  const intptr_t d = reinterpret_cast<intptr_t>(b) - reinterpret_cast<intptr_t>(a);
  if (lda != ldb || d % 2 != 0)
    return overlaps(a, span_bytes(rows, lda, wa), b, span_bytes(rows, ldb, wb));
  const int64_t de = d / 2, ld = lda;
  const int64_t k_lo = std::max<int64_t>(floor_div(de - wa, ld) + 1, -(rows - 1));
  const int64_t k_hi = std::min<int64_t>(floor_div(de + wb - 1, ld), rows - 1);
  for (int64_t k = k_lo; k <= k_hi; ++k) {
    const int64_t t = k * ld;          // t in [de - wa + 1, de + wb - 1] by construction
    if (t > de - wa && t < de + wb) return true;
  }
  return false;
}

}  // namespace

int ds_qk_rows_l2(const uint16_t* q, int64_t ldq, const uint16_t* k, int64_t ldk,
                  const int32_t* positions, const float* inv_freq, const float* q_scale,
                  uint16_t* q_out, int64_t ldq_out, uint16_t* k_out, int64_t ldk_out,
                  int64_t rows, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                  float eps, ds_stream_t stream) {
  if (rows < 0 || n_q_heads < 0 || n_kv_heads < 0) return DS_ERR_SHAPE;
  if (head_dim != 128 && head_dim != 256) return DS_ERR_SHAPE;
  if (!finite_nonneg(eps)) return DS_ERR_ARG;
  const int64_t wq = (int64_t)n_q_heads * head_dim, wk = (int64_t)n_kv_heads * head_dim;
  if (wq > (1 << 24) || wk > (1 << 24)) return DS_ERR_SHAPE;
  if (rows == 0 || wq + wk == 0) return DS_OK;
  if (positions == nullptr || inv_freq == nullptr) return DS_ERR_NULL;
  if (wq > 0 && (q == nullptr || q_out == nullptr || q_scale == nullptr)) return DS_ERR_NULL;
  if (wk > 0 && (k == nullptr || k_out == nullptr)) return DS_ERR_NULL;
  if (wq > 0 && (ldq < wq || ldq_out < wq || ldq % 8 != 0 || ldq_out % 8 != 0)) return DS_ERR_SHAPE;
  if (wk > 0 && (ldk < wk || ldk_out < wk || ldk % 8 != 0 || ldk_out % 8 != 0)) return DS_ERR_SHAPE;
  const int64_t ldmax = std::max(std::max(ldq, ldq_out), std::max(ldk, ldk_out));
  if (rows > (INT64_MAX / 8) / std::max<int64_t>(ldmax, 1)) return DS_ERR_SHAPE;
  if (!aligned(positions, 4) || !aligned(inv_freq, 16) ||
      (wq > 0 && (!aligned(q, 16) || !aligned(q_out, 16) || !aligned(q_scale, 16))) ||
      (wk > 0 && (!aligned(k, 16) || !aligned(k_out, 16))))
    return DS_ERR_ALIGN;
  // outputs: each exactly its input (same stride: in place) or sharing no element with
  // it; never sharing an element with the other input, the other output or the vectors
  // (q and k may be column slices of one fused projection row)
  const size_t bqo = wq > 0 ? span_bytes(rows, ldq_out, wq) : 0;
  const size_t bko = wk > 0 ? span_bytes(rows, ldk_out, wk) : 0;
  auto vectors_clear = [&](const void* out, size_t nb) {
    return !overlaps(out, nb, positions, (size_t)rows * 4) &&
           !overlaps(out, nb, inv_freq, (size_t)head_dim * 2) &&
           !(wq > 0 && overlaps(out, nb, q_scale, (size_t)wq * 4));
  };
  if (wq > 0) {
    const bool in_place = q_out == q && ldq_out == ldq;
    if (!in_place && views_overlap(q_out, ldq_out, wq, q, ldq, wq, rows)) return DS_ERR_ARG;
    if (wk > 0 && views_overlap(q_out, ldq_out, wq, k, ldk, wk, rows)) return DS_ERR_ARG;
    if (!vectors_clear(q_out, bqo)) return DS_ERR_ARG;
  }
  if (wk > 0) {
    const bool in_place = k_out == k && ldk_out == ldk;
    if (!in_place && views_overlap(k_out, ldk_out, wk, k, ldk, wk, rows)) return DS_ERR_ARG;
    if (wq > 0 && views_overlap(k_out, ldk_out, wk, q, ldq, wq, rows)) return DS_ERR_ARG;
    if (!vectors_clear(k_out, bko)) return DS_ERR_ARG;
  }
  if (wq > 0 && wk > 0 && views_overlap(q_out, ldq_out, wq, k_out, ldk_out, wk, rows))
    return DS_ERR_ARG;

  int cus = 0;
  int st = device_cus(&cus);
  if (st != DS_OK) return st;
  dsr::QkArgs a{};
  a.q = q;
  a.k = k;
  a.pos = positions;
  a.inv_freq = inv_freq;
  a.q_scale = q_scale;
  a.qo = q_out;
  a.ko = k_out;
  a.ldq = ldq;
  a.ldk = ldk;
  a.ldqo = ldq_out;
  a.ldko = ldk_out;
  a.rows = rows;
  a.nq = n_q_heads;
  a.nk = n_kv_heads;
  a.eps = eps;
  (void)hipGetLastError();
  const int rpg = dsr::kQkRowsPerBlock;
  return launch_status(launch_in_pieces(rows, rpg, cus, [&](int64_t r0, int64_t n) {
    dsr::QkArgs p = a;
    p.q = q != nullptr ? q + r0 * ldq : nullptr;
    p.k = k != nullptr ? k + r0 * ldk : nullptr;
    p.pos = positions + r0;
    p.qo = q_out != nullptr ? q_out + r0 * ldq_out : nullptr;
    p.ko = k_out != nullptr ? k_out + r0 * ldk_out : nullptr;
    p.rows = n;
    return dsr::launch_qk_rows_l2(head_dim, p, (int)((n + rpg - 1) / rpg), (hipStream_t)stream);
  }));
}

int ds_weight_rownorm_gain(const ds_rownorm_desc* descs, int32_t n, ds_stream_t stream) {
  if (n < 0) return DS_ERR_ARG;
  if (n == 0) return DS_OK;
  if (descs == nullptr) return DS_ERR_NULL;

  // validate every descriptor before anything is enqueued
  std::vector<Range> outs, ins;
  std::vector<std::pair<Shape, dsr::RownormTask>> mats;
  for (int32_t i = 0; i < n; ++i) {
    const ds_rownorm_desc& d = descs[i];
    Shape s;
    uintptr_t a32 = 16, a16 = 16;
    int64_t span = 0;
    int st = check_layout(d.rows, d.cols, d.seg, d.ld, &s, &a32, &a16, &span);
    if (st != DS_OK) return st;
    if (!std::isfinite(d.radius) || !gain_mode_ok(d.gain_mode)) return DS_ERR_ARG;
    if (d.rows == 0) continue;
    const float* gain = d.gain_mode == DS_GAIN_NONE ? nullptr : d.gain;
    if (d.w == nullptr || d.w_eff == nullptr || (d.gain_mode != DS_GAIN_NONE && gain == nullptr))
      return DS_ERR_NULL;
    if (!aligned(d.w, a32) || !aligned(d.w_eff, a16) || !aligned(gain, 4) ||
        (d.norm_out != nullptr && !aligned(d.norm_out, 4)))
      return DS_ERR_ALIGN;
    const size_t nel = (size_t)span;
    add_range(ins, d.w, nel * 4);
    add_range(ins, gain, gain_bytes(d.gain_mode, d.rows));
    add_range(outs, d.w_eff, nel * 2);
    add_range(outs, d.norm_out, (size_t)d.rows * 4);
    dsr::RownormTask t{};
    t.w = d.w;
    t.gain = gain;
    t.gain_stride = d.gain_mode == DS_GAIN_ROW ? 1 : 0;
    t.norm_out = d.norm_out;
    t.w_eff = d.w_eff;
    t.rows = d.rows;
    t.cols = (int32_t)d.cols;
    t.radius = d.radius;
    t.seg = d.seg;
    t.ld = d.ld;
    s = single_pass(s, dsr::kCol1KFwd, dsr::kCol1LanesFwd, d.rows, d.cols, d.seg, d.ld,
                    aligned(d.w, 16) && aligned(d.w_eff, 8));
    mats.emplace_back(s, t);
  }
  if (!outputs_disjoint(outs, ins)) return DS_ERR_ARG;
  return launch_ragged<dsr::RownormTask>(mats, launch_rownorm_any, (hipStream_t)stream);
}

int ds_l2_rows_backward(const uint16_t* x, const uint16_t* r, const uint16_t* dy, uint16_t* dx,
                        int64_t rows, int64_t cols, float eps, ds_stream_t stream) {
  return norm_rows_backward(dsr::launch_l2_rows_backward, x, r, dy, dx, rows, cols, eps, stream);
}

int ds_rms_rows_backward(const uint16_t* x, const uint16_t* r, const uint16_t* dy, uint16_t* dx,
                         int64_t rows, int64_t cols, float eps, ds_stream_t stream) {
  return norm_rows_backward(dsr::launch_rms_rows_backward, x, r, dy, dx, rows, cols, eps, stream);
}

namespace {

// ------------------------------------------------------- library scratch
//
// The allocation-free weight gradient keeps a scalar gain's per-row shares
// here instead of in a caller's buffer.  Each device holds its own copy of
// the array until the process ends.  In host code `scratch` names a host
// stand-in, not device memory: host code uses only the address that
// hipGetSymbolAddress returns for the current device, fetched once per device
// and kept.  Every call on a device shares that device's array; it is
// written (every share) before it is read, so nothing is cleared.

__device__ __align__(256) float scratch[DS_SCRATCH_FLOATS];

int scratch_for_current_device(float** out) {
  static std::mutex mu;
  static std::map<int, float*> ptrs;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return DS_ERR_DEVICE;
  std::lock_guard<std::mutex> lock(mu);
  auto it = ptrs.find(dev);
  if (it == ptrs.end()) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr)
      return DS_ERR_DEVICE;
    it = ptrs.emplace(dev, static_cast<float*>(p)).first;
  }
  *out = it->second;
  return DS_OK;
}

// The weight gradient.  `noalloc`: a scalar gain's shares go to the library
// scratch (its descriptor's dgain must be NULL) and every launch carries its
// table in the kernel arguments, so the call allocates nothing.
int rownorm_backward_call(const ds_rownorm_grad_desc* descs, int32_t n, ds_stream_t stream,
                          bool noalloc) {
  if (n < 0) return DS_ERR_ARG;
  if (n == 0) return DS_OK;
  if (descs == nullptr) return DS_ERR_NULL;

  std::vector<Range> outs, ins;
  std::vector<std::pair<Shape, dsr::RownormGradTask>> mats;
  std::vector<dsr::TotalTask> totals;
  std::vector<std::pair<size_t, int64_t>> scratch_users;   // (task in mats, offset in scratch)
  std::vector<std::pair<size_t, int64_t>> scratch_totals;  // (entry in totals, offset)
  int64_t scratch_used = 0;
  for (int32_t i = 0; i < n; ++i) {
    const ds_rownorm_grad_desc& d = descs[i];
    Shape s;
    uintptr_t a32 = 16, a16 = 16;
    int64_t span = 0;
    int st = check_layout(d.rows, d.cols, d.seg, d.ld, &s, &a32, &a16, &span);
    if (st != DS_OK) return st;
    if (!std::isfinite(d.radius) || !gain_mode_ok(d.gain_mode)) return DS_ERR_ARG;
    const bool shares_in_scratch = noalloc && d.gain_mode == DS_GAIN_SCALAR;
    if (shares_in_scratch && d.dgain != nullptr) return DS_ERR_ARG;
    // a total needs a scalar gain and the per-row shares it sums (none for an
    // empty matrix); no gain, no gradient
    if (d.dgain_total != nullptr &&
        (d.gain_mode != DS_GAIN_SCALAR ||
         (!shares_in_scratch && d.dgain == nullptr && d.rows > 0)))
      return DS_ERR_ARG;
    if (d.gain_mode == DS_GAIN_NONE && d.dgain != nullptr) return DS_ERR_ARG;
    if (d.rows == 0) {
      // the sum over no rows: the total kernel writes 0 and reads nothing
      if (d.dgain_total != nullptr) {
        if (!aligned(d.dgain_total, 4)) return DS_ERR_ALIGN;
        add_range(outs, d.dgain_total, 4);
        totals.push_back({d.dgain, d.dgain_total, 0});
      }
      continue;
    }
    const float* gain = d.gain_mode == DS_GAIN_NONE ? nullptr : d.gain;
    if (d.w == nullptr || d.dw_eff == nullptr || d.dw == nullptr ||
        (d.gain_mode != DS_GAIN_NONE && gain == nullptr))
      return DS_ERR_NULL;
    if (!aligned(d.w, a32) || !aligned(d.dw_eff, a16) || !aligned(d.dw, a32) ||
        !aligned(gain, 4) || !aligned(d.dgain, 4) || !aligned(d.dgain_total, 4))
      return DS_ERR_ALIGN;
    const size_t nel = (size_t)span;
    add_range(ins, d.w, nel * 4);
    add_range(ins, gain, gain_bytes(d.gain_mode, d.rows));
    add_range(ins, d.dw_eff, nel * 2);
    add_range(outs, d.dw, nel * 4);
    add_range(outs, d.dgain, (size_t)d.rows * 4);
    add_range(outs, d.dgain_total, 4);
    dsr::RownormGradTask t{};
    t.w = d.w;
    t.gain = gain;
    t.gain_stride = d.gain_mode == DS_GAIN_ROW ? 1 : 0;
    t.dw_eff = d.dw_eff;
    t.dw = d.dw;
    t.dgain = d.dgain;
    t.rows = d.rows;
    t.cols = (int32_t)d.cols;
    t.radius = d.radius;
    t.seg = d.seg;
    t.ld = d.ld;
    if (shares_in_scratch && d.dgain_total != nullptr) {
      if (d.rows > DS_SCRATCH_FLOATS - scratch_used) return DS_ERR_SCRATCH;
      scratch_users.emplace_back(mats.size(), scratch_used);
      scratch_totals.emplace_back(totals.size(), scratch_used);
      scratch_used += d.rows;
    }
    if (d.dgain_total != nullptr) totals.push_back({d.dgain, d.dgain_total, d.rows});
    s = single_pass(s, dsr::kCol1KBwd, dsr::kCol1LanesBwd, d.rows, d.cols, d.seg, d.ld,
                    aligned(d.w, 16) && aligned(d.dw_eff, 8) && aligned(d.dw, 16));
    mats.emplace_back(s, t);
  }
  if (!outputs_disjoint(outs, ins)) return DS_ERR_ARG;
  if (!scratch_users.empty()) {
    float* sp = nullptr;
    int st = scratch_for_current_device(&sp);
    if (st != DS_OK) return st;
    for (auto& u : scratch_users) mats[u.first].second.dgain = sp + u.second;
    for (auto& u : scratch_totals) totals[u.first].shares = sp + u.second;
  }
  int st = launch_ragged<dsr::RownormGradTask>(mats, launch_rownorm_backward_any,
                                               (hipStream_t)stream, noalloc);
  if (st != DS_OK) return st;
  if (!totals.empty()) {                          // (a call of empty matrices has no launch above)
    int cus = 0;
    if ((st = device_cus(&cus)) != DS_OK) return st;
  }
  // scalar gains: sum each matrix's row shares once the shares are written
  for (size_t first = 0; first < totals.size(); first += dsr::kTotalTasks) {
    dsr::TotalArgs args{};
    args.ntasks = (int32_t)std::min<size_t>(dsr::kTotalTasks, totals.size() - first);
    for (int k = 0; k < args.ntasks; ++k) args.tasks[k] = totals[first + k];
    dsr::row_total_kernel<<<args.ntasks, 256, 0, (hipStream_t)stream>>>(args);
    if (hipGetLastError() != hipSuccess) return DS_ERR_LAUNCH;
  }
  return DS_OK;
}

}  // namespace

int ds_weight_rownorm_gain_backward(const ds_rownorm_grad_desc* descs, int32_t n,
                                    ds_stream_t stream) {
  return rownorm_backward_call(descs, n, stream, false);
}

int ds_weight_rownorm_gain_backward_noalloc(const ds_rownorm_grad_desc* descs, int32_t n,
                                            ds_stream_t stream) {
  return rownorm_backward_call(descs, n, stream, true);
}

namespace {

// The rescale method's ragged calls: `project` writes v only (w is read);
// `after_step` writes w and, when given, v.
int rescale_call(const ds_rescale_desc* descs, int32_t n, bool after_step, ds_stream_t stream) {
  if (n < 0) return DS_ERR_ARG;
  if (n == 0) return DS_OK;
  if (descs == nullptr) return DS_ERR_NULL;
  std::vector<Range> outs, ins;
  std::vector<std::pair<Shape, dsr::RescaleTask>> mats;
  for (int32_t i = 0; i < n; ++i) {
    const ds_rescale_desc& d = descs[i];
    Shape s;
    uintptr_t a32 = 16, a16 = 16;
    int64_t span = 0;
    int st = check_layout(d.rows, d.cols, d.seg, d.ld, &s, &a32, &a16, &span);
    if (st != DS_OK) return st;
    if (after_step && !std::isfinite(d.radius)) return DS_ERR_ARG;
    if (d.rows == 0) continue;
    if (d.w == nullptr || (!after_step && d.v == nullptr)) return DS_ERR_NULL;
    if (!aligned(d.w, a32) || !aligned(d.v, a32)) return DS_ERR_ALIGN;
    const size_t nb = (size_t)span * 4;
    add_range(after_step ? outs : ins, d.w, nb);
    add_range(outs, d.v, nb);
    dsr::RescaleTask t{};
    t.w = d.w;
    t.v = d.v;
    t.rows = d.rows;
    t.cols = (int32_t)d.cols;
    t.radius = d.radius;
    t.seg = d.seg;
    t.ld = d.ld;
    s = single_pass(s, dsr::kCol1KRescale, dsr::kCol1LanesRescale, d.rows, d.cols, d.seg, d.ld,
                    aligned(d.w, 16) && aligned(d.v, 16));
    mats.emplace_back(s, t);
  }
  if (!outputs_disjoint(outs, ins)) return DS_ERR_ARG;
  return launch_ragged<dsr::RescaleTask>(
      mats, after_step ? launch_after_step_any : launch_project_any, (hipStream_t)stream);
}

}  // namespace

int ds_rescale_project(const ds_rescale_desc* descs, int32_t n, ds_stream_t stream) {
  return rescale_call(descs, n, false, stream);
}

int ds_rescale_after_step(const ds_rescale_desc* descs, int32_t n, ds_stream_t stream) {
  return rescale_call(descs, n, true, stream);
}

}  // extern "C"
