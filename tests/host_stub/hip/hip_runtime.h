// Host-only stand-in for <hip/hip_runtime.h>, for building the library's
// host runtime (sv_runtime.cpp) with g++ and no GPU: the HIP types and the
// few API calls the runtime makes, implemented on host memory in
// host_stubs.cpp.  Test infrastructure only; nothing here reaches the HIP
// library.
#pragma once
#include <stddef.h>
#include <stdint.h>

#define __device__
#define __host__
#define __forceinline__ inline
#define __align__(n) __attribute__((aligned(n)))
#define HIP_SYMBOL(x) (reinterpret_cast<const void*>(&(x)))

typedef enum {
  hipSuccess = 0,
  hipErrorInvalidValue = 1,
  hipErrorNotSupported = 801,
  hipErrorUnknown = 999
} hipError_t;

typedef struct ihipStream_t* hipStream_t;
typedef struct ihipGraph_t* hipGraph_t;
typedef struct ihipGraphExec_t* hipGraphExec_t;
typedef struct ihipGraphNode_t* hipGraphNode_t;

struct float2 { float x, y; };
struct int2 { int x, y; };
inline int2 make_int2(int x, int y) { return int2{x, y}; }

enum hipMemcpyKind { hipMemcpyHostToHost = 0, hipMemcpyHostToDevice, hipMemcpyDeviceToHost, hipMemcpyDeviceToDevice };
enum hipDeviceAttribute_t { hipDeviceAttributeMultiprocessorCount = 1, hipDeviceAttributeWallClockRate = 2 };
enum hipStreamCaptureMode { hipStreamCaptureModeGlobal = 0, hipStreamCaptureModeThreadLocal, hipStreamCaptureModeRelaxed };
constexpr unsigned hipHostMallocDefault = 0, hipHostMallocMapped = 2, hipHostMallocCoherent = 0x40000000;
constexpr unsigned hipStreamNonBlocking = 1;

hipError_t hipGetDevice(int* dev);
hipError_t hipDeviceGetAttribute(int* v, hipDeviceAttribute_t attr, int dev);
hipError_t hipGetSymbolAddress(void** p, const void* symbol);
hipError_t hipHostMalloc(void** p, size_t bytes, unsigned flags);
hipError_t hipHostFree(void* p);
hipError_t hipHostGetDevicePointer(void** dev, void* host, unsigned flags);
hipError_t hipMemcpy(void* dst, const void* src, size_t bytes, hipMemcpyKind kind);
hipError_t hipMemcpyAsync(void* dst, const void* src, size_t bytes, hipMemcpyKind kind, hipStream_t st);
hipError_t hipStreamCreateWithFlags(hipStream_t* st, unsigned flags);
hipError_t hipStreamDestroy(hipStream_t st);
hipError_t hipStreamSynchronize(hipStream_t st);
hipError_t hipStreamBeginCapture(hipStream_t st, hipStreamCaptureMode mode);
hipError_t hipStreamEndCapture(hipStream_t st, hipGraph_t* graph);
hipError_t hipGraphInstantiate(hipGraphExec_t* exec, hipGraph_t graph, hipGraphNode_t* err_node, char* log,
                               size_t log_size);
hipError_t hipGraphLaunch(hipGraphExec_t exec, hipStream_t st);
hipError_t hipGraphDestroy(hipGraph_t graph);
hipError_t hipGraphExecDestroy(hipGraphExec_t exec);
