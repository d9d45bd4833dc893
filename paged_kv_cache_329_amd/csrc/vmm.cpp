// A KV pool in contiguous virtual memory backed on demand (the alternative the pages weigh
// against paging: "What is PagedAttention?" (qubittool glossary), "Frequently Asked
// Questions" and "Common Use Cases", contrasting paged blocks with contiguous virtual
// memory whose physical pages are mapped as a sequence grows).
//
// The virtual range of each of the K and V pools is reserved once.  Sequence s owns a
// contiguous slice of max_blocks_per_seq blocks starting at a page boundary; physical
// memory is created and mapped page by page (hipMemCreate / hipMemMap / hipMemSetAccess)
// as the sequence grows, and unmapped and released when it ends.  A page holds whole
// blocks and whole device granules.  The slice's blocks keep the pool layout of
// include/pagedkv.h, so the attention kernels read this pool unchanged, with block tables
// that count up from the slice's first block.
//
// The first page of each pool is mapped for the pool's lifetime (block 0 lives there):
// the kernels read block 0 in place of a table entry outside the pool, so it must always be
// backed.  Sequence slices start after it.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <vector>

#include "status.h"

struct pkv_vmm {
  int device = 0;
  int max_seqs = 0;
  int max_blocks = 0;            // per sequence
  size_t block_bytes = 0;        // one block of one pool (all kv heads)
  size_t gran = 0;               // mapping unit ("page"): whole blocks, a multiple of the
                                 // device's minimum granule
  size_t slice_bytes = 0;        // a sequence's virtual slice, a multiple of gran
  size_t base_bytes = 0;         // the always-mapped first page
  size_t total_bytes = 0;        // per pool
  void* va[2] = {nullptr, nullptr};                                  // K, V
  std::vector<std::vector<hipMemGenericAllocationHandle_t>> mapped;  // [seq] pages, K then V
  hipMemGenericAllocationHandle_t base_handle[2] = {};
  size_t mapped_bytes = 0;       // physical bytes mapped, both pools, base included
};

namespace {

using pkv::fail;

hipMemAllocationProp device_prop(int device) {
  hipMemAllocationProp prop;
  std::memset(&prop, 0, sizeof(prop));
  prop.type = hipMemAllocationTypePinned;
  prop.location.type = hipMemLocationTypeDevice;
  prop.location.id = device;
  return prop;
}

// Creates one page of physical memory and maps it read-write at `at`; on failure nothing
// stays mapped.
pkv_status map_granule(const pkv_vmm* v, char* at, hipMemGenericAllocationHandle_t* out) {
  const hipMemAllocationProp prop = device_prop(v->device);
  hipMemGenericAllocationHandle_t h;
  hipError_t e = hipMemCreate(&h, v->gran, &prop, 0);
  if (e != hipSuccess) return fail(PKV_OUT_OF_BLOCKS, "pkv_vmm: hipMemCreate: %s", hipGetErrorString(e));
  e = hipMemMap(at, v->gran, 0, h, 0);
  if (e != hipSuccess) {
    (void)hipMemRelease(h);
    return fail(PKV_HIP_ERROR, "pkv_vmm: hipMemMap: %s", hipGetErrorString(e));
  }
  hipMemAccessDesc desc;
  std::memset(&desc, 0, sizeof(desc));
  desc.location = prop.location;
  desc.flags = hipMemAccessFlagsProtReadWrite;
  e = hipMemSetAccess(at, v->gran, &desc, 1);
  if (e != hipSuccess) {
    (void)hipMemUnmap(at, v->gran);
    (void)hipMemRelease(h);
    return fail(PKV_HIP_ERROR, "pkv_vmm: hipMemSetAccess: %s", hipGetErrorString(e));
  }
  *out = h;
  return PKV_OK;
}

void unmap_granule(const pkv_vmm* v, char* at, hipMemGenericAllocationHandle_t h) {
  (void)hipMemUnmap(at, v->gran);
  (void)hipMemRelease(h);
}

char* slice(const pkv_vmm* v, int pool, int seq) {
  return static_cast<char*>(v->va[pool]) + v->base_bytes + size_t(seq) * v->slice_bytes;
}

// Waits for all work on the pool's device, so that no kernel still in flight reads pages
// about to be unmapped (an unmapped address faults the GPU).  The caller's current device is
// kept.
hipError_t drain(const pkv_vmm* v) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != v->device && (e = hipSetDevice(v->device)) != hipSuccess) return e;
  e = hipDeviceSynchronize();
  if (cur != v->device) (void)hipSetDevice(cur);
  return e;
}

void destroy(pkv_vmm* v) {
  (void)drain(v);
  for (int s = 0; s < int(v->mapped.size()); ++s) {
    auto& hs = v->mapped[s];
    const size_t n = hs.size() / 2;
    for (size_t g = 0; g < n; ++g) {
      unmap_granule(v, slice(v, 0, s) + g * v->gran, hs[g]);
      unmap_granule(v, slice(v, 1, s) + g * v->gran, hs[n + g]);
    }
  }
  for (int p = 0; p < 2; ++p) {
    if (v->base_handle[p]) unmap_granule(v, static_cast<char*>(v->va[p]), v->base_handle[p]);
    if (v->va[p]) (void)hipMemAddressFree(v->va[p], v->total_bytes);
  }
  delete v;
}

}  // namespace

extern "C" {

pkv_vmm* pkv_vmm_create(int device, int max_seqs, int max_blocks_per_seq, size_t block_bytes,
                        size_t page_bytes) {
  if (max_seqs <= 0 || max_blocks_per_seq <= 0 || block_bytes == 0 || block_bytes % 16) {
    fail(PKV_INVALID_ARG, "pkv_vmm_create: max_seqs=%d max_blocks_per_seq=%d block_bytes=%zu", max_seqs,
         max_blocks_per_seq, block_bytes);
    return nullptr;
  }
  auto* v = new (std::nothrow) pkv_vmm;
  if (!v) {
    fail(PKV_INVALID_ARG, "pkv_vmm_create: out of host memory");
    return nullptr;
  }
  v->device = device;
  v->max_seqs = max_seqs;
  v->max_blocks = max_blocks_per_seq;
  v->block_bytes = block_bytes;
  const hipMemAllocationProp prop = device_prop(device);
  size_t gmin = 0, grec = 0;
  hipError_t e = hipMemGetAllocationGranularity(&gmin, &prop, hipMemAllocationGranularityMinimum);
  if (e == hipSuccess) e = hipMemGetAllocationGranularity(&grec, &prop, hipMemAllocationGranularityRecommended);
  if (e != hipSuccess || gmin == 0) {
    fail(PKV_UNSUPPORTED, "pkv_vmm_create: no virtual memory management on device %d (%s)", device,
         hipGetErrorString(e));
    delete v;
    return nullptr;
  }
  // The mapping unit holds whole blocks and whole granules: a multiple of lcm(granule,
  // block), at least the requested size (default: the runtime's recommended granule).
  size_t a = gmin, b = block_bytes;
  while (b) {
    const size_t t = a % b;
    a = b;
    b = t;
  }
  const size_t unit = gmin / a * block_bytes;
  const size_t want = std::max<size_t>(page_bytes ? page_bytes : std::max<size_t>(grec, gmin), unit);
  v->gran = (want + unit - 1) / unit * unit;
  v->slice_bytes = (size_t(max_blocks_per_seq) * block_bytes + v->gran - 1) / v->gran * v->gran;
  v->base_bytes = v->gran;
  v->total_bytes = v->base_bytes + size_t(max_seqs) * v->slice_bytes;
  if (v->total_bytes / block_bytes > size_t(INT32_MAX)) {
    fail(PKV_UNSUPPORTED, "pkv_vmm_create: more than 2^31 virtual blocks");
    delete v;
    return nullptr;
  }
  v->mapped.resize(max_seqs);
  for (int p = 0; p < 2; ++p) {
    e = hipMemAddressReserve(&v->va[p], v->total_bytes, gmin, nullptr, 0);
    if (e != hipSuccess) {
      v->va[p] = nullptr;
      fail(PKV_UNSUPPORTED, "pkv_vmm_create: hipMemAddressReserve of %zu bytes: %s", v->total_bytes,
           hipGetErrorString(e));
      destroy(v);
      return nullptr;
    }
    if (map_granule(v, static_cast<char*>(v->va[p]), &v->base_handle[p]) != PKV_OK) {
      destroy(v);
      return nullptr;
    }
    v->mapped_bytes += v->gran;
  }
  // Block 0 (and the rest of the base page) reads as zeros.
  for (int p = 0; p < 2; ++p) {
    if (hipMemset(v->va[p], 0, v->gran) != hipSuccess) {
      fail(PKV_HIP_ERROR, "pkv_vmm_create: clearing the base page failed");
      destroy(v);
      return nullptr;
    }
  }
  return v;
}

void pkv_vmm_destroy(pkv_vmm* v) {
  if (v) destroy(v);
}

pkv_status pkv_vmm_reserve(pkv_vmm* v, int seq, int num_blocks) {
  if (!v) return fail(PKV_INVALID_ARG, "pkv_vmm_reserve: null pool");
  if (seq < 0 || seq >= v->max_seqs || num_blocks < 0 || num_blocks > v->max_blocks)
    return fail(PKV_INVALID_ARG, "pkv_vmm_reserve: seq=%d num_blocks=%d (max %d, %d)", seq, num_blocks,
                v->max_seqs, v->max_blocks);
  auto& hs = v->mapped[seq];
  const size_t have = hs.size() / 2;
  const size_t need = (size_t(num_blocks) * v->block_bytes + v->gran - 1) / v->gran;
  if (need <= have) return PKV_OK;
  std::vector<hipMemGenericAllocationHandle_t> k(hs.begin(), hs.begin() + have), vv(hs.begin() + have, hs.end());
  for (size_t g = have; g < need; ++g) {
    hipMemGenericAllocationHandle_t hk, hv;
    pkv_status st = map_granule(v, slice(v, 0, seq) + g * v->gran, &hk);
    if (st == PKV_OK) {
      st = map_granule(v, slice(v, 1, seq) + g * v->gran, &hv);
      if (st != PKV_OK) unmap_granule(v, slice(v, 0, seq) + g * v->gran, hk);
    }
    if (st != PKV_OK) {
      // All-or-nothing: drop what this call mapped.
      for (size_t r = have; r < g; ++r) {
        unmap_granule(v, slice(v, 0, seq) + r * v->gran, k[r]);
        unmap_granule(v, slice(v, 1, seq) + r * v->gran, vv[r]);
      }
      return st;
    }
    k.push_back(hk);
    vv.push_back(hv);
  }
  v->mapped_bytes += 2 * (need - have) * v->gran;
  hs = std::move(k);
  hs.insert(hs.end(), vv.begin(), vv.end());
  return PKV_OK;
}

pkv_status pkv_vmm_release(pkv_vmm* v, int seq) {
  if (!v) return fail(PKV_INVALID_ARG, "pkv_vmm_release: null pool");
  if (seq < 0 || seq >= v->max_seqs) return fail(PKV_INVALID_ARG, "pkv_vmm_release: seq=%d", seq);
  auto& hs = v->mapped[seq];
  const size_t n = hs.size() / 2;
  if (n == 0) return PKV_OK;
  const hipError_t e = drain(v);
  if (e != hipSuccess)
    return fail(PKV_HIP_ERROR, "pkv_vmm_release: synchronising the device: %s", hipGetErrorString(e));
  for (size_t g = 0; g < n; ++g) {
    unmap_granule(v, slice(v, 0, seq) + g * v->gran, hs[g]);
    unmap_granule(v, slice(v, 1, seq) + g * v->gran, hs[n + g]);
  }
  v->mapped_bytes -= 2 * n * v->gran;
  hs.clear();
  return PKV_OK;
}

void* pkv_vmm_k_base(const pkv_vmm* v) { return v ? v->va[0] : nullptr; }
void* pkv_vmm_v_base(const pkv_vmm* v) { return v ? v->va[1] : nullptr; }
int pkv_vmm_num_blocks(const pkv_vmm* v) { return v ? int(v->total_bytes / v->block_bytes) : -1; }
int pkv_vmm_seq_first_block(const pkv_vmm* v, int seq) {
  if (!v || seq < 0 || seq >= v->max_seqs) return -1;
  return int((v->base_bytes + size_t(seq) * v->slice_bytes) / v->block_bytes);
}
int pkv_vmm_mapped_blocks(const pkv_vmm* v, int seq) {
  if (!v || seq < 0 || seq >= v->max_seqs) return -1;
  return int(v->mapped[seq].size() / 2 * v->gran / v->block_bytes);
}
size_t pkv_vmm_mapped_bytes(const pkv_vmm* v) { return v ? v->mapped_bytes : 0; }
size_t pkv_vmm_page_bytes(const pkv_vmm* v) { return v ? v->gran : 0; }

}  // extern "C"
