// Registry of the caller-side regions (tensors, workspace) the launch stubs
// check device pointers against; shared by the sanitizer driver and stubs.
#pragma once
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif
void sanitize_reset(void);
void sanitize_region(const void* base, int64_t bytes);
int sanitize_calls(void);
int sanitize_violations(void);
#ifdef __cplusplus
}
#endif
