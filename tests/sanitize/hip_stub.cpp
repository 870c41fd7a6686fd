// A stand-in for the HIP runtime with no device, for the sanitized host
// build of the GPU library (tests/test_sanitize_cpu.py): every call that
// would reach a device reports that there is none, kernel registration does
// nothing, and no kernel can be launched.  Only the runtime functions the
// library's host code refers to are defined; their argument types do not
// matter to the linker (C linkage), only that none of them is reached with
// a device expected.
#include <cstddef>

extern "C" {

enum { kNoDevice = 100, kInvalidValue = 1 };   // hipErrorNoDevice, hipErrorInvalidValue

static int g_last = 0;

int hipGetDeviceCount(int *count)
{
    if (count) *count = 0;
    return g_last = kNoDevice;
}
int hipGetDevice(int *dev)
{
    if (dev) *dev = -1;
    return g_last = kNoDevice;
}
int hipGetDevicePropertiesR0600(void *, int) { return g_last = kNoDevice; }
int hipGetLastError(void)
{
    const int e = g_last;
    g_last = 0;
    return e;
}
int hipGetSymbolAddress(void **p, const void *)
{
    if (p) *p = nullptr;
    return g_last = kNoDevice;
}
int hipMallocAsync(void **p, size_t, void *)
{
    if (p) *p = nullptr;
    return g_last = kNoDevice;
}
int hipFreeAsync(void *, void *) { return g_last = kNoDevice; }
int hipLaunchKernel(const void *, ...) { return g_last = kNoDevice; }
int __hipPushCallConfiguration(...) { return 0; }
int __hipPopCallConfiguration(...) { return 0; }

static int g_handle;
void **__hipRegisterFatBinary(const void *) { return reinterpret_cast<void **>(&g_handle); }
void __hipUnregisterFatBinary(void **) {}
void __hipRegisterFunction(...) {}
void __hipRegisterVar(...) {}

}  // extern "C"
