// Per-kernel resources from the compiler's report of this build (registers,
// scratch, LDS, the occupancy they allow): the residency facts of "GPU
// 算子优化中的数据复用", sections 9 (spills) and 12 (resident blocks are the
// minimum over the limits).  The build script parses the report of the
// kernel units and writes the table (kernel_resources.cpp in the build
// folder), keyed by each kernel's mangled name; the host finds a kernel's
// name from its handle with dladdr.
#pragma once

namespace gemmf32 {

struct KernelResources {
    const char *name;     // mangled kernel name
    int vgprs;            // architectural vector registers per lane
    int agprs;            // accumulation registers per lane
    int sgprs;            // scalar registers per wavefront
    int scratch_bytes;    // private memory per lane (register spills)
    int lds_bytes;        // LDS per workgroup
    int waves_per_simd;   // the compiler's occupancy estimate
};

extern const KernelResources kKernelResources[];
extern const int kKernelResourcesCount;

}  // namespace gemmf32
