// Internal: the calling thread's last-error text behind pa_last_error().
#pragma once

// Record a formatted message for pa_last_error() and return `status`.
int pa_fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
// Clear the message and return PA_OK.
int pa_ok();
